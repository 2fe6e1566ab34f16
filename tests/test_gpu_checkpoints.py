"""GPU: chunk-boundary state checkpoints (gdr_chunk_fwd_checkpoints) against
the oracle's per-chunk states, and o / ht against the plain entry point.

Chunk c of sequence n holds its tokens 64c .. min(64(c+1), L_n) - 1; its row
is sum(ceil(L_m / 64), m < n) + c and receives the state after the last of
them.  Tolerance: that of ht (2e-2 absolute for bf16 inputs, 2e-5 for f32
inputs; the states are ht-like).  Rows past the true chunk count keep the
caller's sentinel.
"""
import numpy as np
import pytest

import gdr_inputs as gi
from gpu_helpers import compare, np64, run_gpu, say, to_device, tols

pytestmark = pytest.mark.gpu


def _oracle_chunks(d):
    import oracle
    return oracle.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["h0"],
                          scale=d["scale"], chunk_states=True)


def _run(t, d, rows, sentinel=7.0):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    cu = t["cu"]
    N = (cu.shape[0] - 1) if cu is not None else t["q"].shape[0]
    hv, dk = t["v"].shape[2], t["q"].shape[3]
    hck = torch.full((rows, hv, dk, dk), sentinel, dtype=torch.float32, device="cuda")
    ht = torch.zeros((N, hv, dk, dk), dtype=torch.float32, device="cuda")
    o, ht, hck = gdr.chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, t["h0"],
                                           scale=d["scale"], ht=ht, h_chunks=hck)
    torch.cuda.synchronize()
    return o, ht, hck


def _check(t, d, rows, what):
    o, ht, hck = _run(t, d, rows)
    o_ref, ht_ref, hck_ref = _oracle_chunks(d)
    nt = hck_ref.shape[0]
    tol_o, tol_ht = tols(d["dtype"])
    compare(o, ht, o_ref, ht_ref, what, tol_o, tol_ht)
    got = np64(hck)
    err = float(np.abs(got[:nt] - hck_ref).max())
    say("%s: %d chunk states, max|dh_chunk| %.3e (max_ref %.4f)" % (what, nt, err, float(np.abs(hck_ref).max())))
    assert np.all(np.isfinite(got[:nt]))
    assert err <= tol_ht
    assert np.all(got[nt:] == 7.0), "rows past the chunk count were written"
    # the plain entry point gives the same o and ht, bit for bit
    o2, ht2 = run_gpu(t, d["scale"])
    assert np.array_equal(np64(o), np64(o2)), "o differs from gdr_chunk_fwd"
    assert np.array_equal(np64(ht), np64(ht2)), "ht differs from gdr_chunk_fwd"


@pytest.mark.parametrize("d_head,dtype,hk,hv", [(128, "bf16", 2, 4), (64, "fp32", 1, 2), (128, "fp32", 2, 2)])
def test_checkpoints_ragged(d_head, dtype, hk, hv):
    lens = [1, 63, 0, 64, 65, 127, 0, 128, 129, 200, 0]
    say("checkpoints ragged: d=%d %s Hk=%d Hv=%d" % (d_head, dtype, hk, hv))
    w = gi.Workload("ragged", 1, 0, hk, hv, d_head, d_head, dtype, seg_range=(1, 2),
                    n_segments=len(lens), seed=91)
    d = gi.generate(w, lengths=lens)
    t = to_device(d)
    rows = (sum(lens) + 63) // 64 + len(lens)
    _check(t, d, rows, "ckpt ragged d=%d %s" % (d_head, dtype))


def test_checkpoints_fixed_length():
    say("checkpoints fixed B=4 T=512")
    d = gi.generate(gi.WORKLOADS["fixed_B4_T512_H16_d128"])
    t = to_device(d)
    _check(t, d, 4 * 8, "ckpt fixed B4 T512")


def test_checkpoints_tiny():
    say("checkpoints tiny")
    d = gi.generate(gi.WORKLOADS["tiny_fp32_T128_H2_d64"])
    t = to_device(d)
    _check(t, d, 2, "ckpt tiny")
