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
    hv, dk, dv = t["v"].shape[2], t["q"].shape[3], t["v"].shape[3]
    hck = torch.full((rows, hv, dk, dv), sentinel, dtype=torch.float32, device="cuda")
    ht = torch.zeros((N, hv, dk, dv), dtype=torch.float32, device="cuda")
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


# ---------------------------------------------------------------------------
# Checkpoints every n tokens (gdr_chunk_fwd_checkpoints_n)
# ---------------------------------------------------------------------------

def _run_n(t, d, rows, every, sentinel=7.0):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    cu = t["cu"]
    N = (cu.shape[0] - 1) if cu is not None else t["q"].shape[0]
    hv, dk, dv = t["v"].shape[2], t["q"].shape[3], t["v"].shape[3]
    hck = torch.full((rows, hv, dk, dv), sentinel, dtype=torch.float32, device="cuda")
    ht = torch.zeros((N, hv, dk, dv), dtype=torch.float32, device="cuda")
    o, ht, hck = gdr.chunk_fwd_checkpoints(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, t["h0"],
                                           scale=d["scale"], ht=ht, h_chunks=hck, every_n=every)
    torch.cuda.synchronize()
    return o, ht, hck


def _check_n(t, d, rows, every, what):
    import oracle
    o, ht, hck = _run_n(t, d, rows, every)
    o_ref, ht_ref, hck_ref = oracle.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                            d["h0"], scale=d["scale"], chunk_states=True,
                                            checkpoint_every=every)
    nt = hck_ref.shape[0]
    tol_o, tol_ht = tols(d["dtype"])
    compare(o, ht, o_ref, ht_ref, what, tol_o, tol_ht)
    got = np64(hck)
    err = float(np.abs(got[:nt] - hck_ref).max())
    say("%s: %d checkpoint rows (every %d), max|dh_ckpt| %.3e (max_ref %.4f)"
        % (what, nt, every, err, float(np.abs(hck_ref).max())))
    assert np.all(np.isfinite(got[:nt]))
    assert err <= tol_ht
    assert np.all(got[nt:] == 7.0), "rows past the checkpoint count were written"
    o2, ht2 = run_gpu(t, d["scale"])
    assert np.array_equal(np64(o), np64(o2)), "o differs from gdr_chunk_fwd"
    assert np.array_equal(np64(ht), np64(ht2)), "ht differs from gdr_chunk_fwd"
    return got[:nt]


@pytest.mark.parametrize("every,d_head,dtype,hk,hv", [
    (16, 128, "bf16", 2, 4), (48, 64, "bf16", 1, 2), (80, 128, "bf16", 1, 1), (128, 128, "bf16", 2, 2),
    (16, 64, "fp32", 1, 2), (32, 128, "fp32", 2, 2)])
def test_checkpoints_every_n_ragged(every, d_head, dtype, hk, hv):
    """Lengths around 16 and 64 (with ghosts), checkpoints every n tokens:
    inside chunks (n = 16, 48, 80), at chunk ends (n = 128), fp32 inputs."""
    lens = [1, 15, 16, 17, 0, 63, 64, 65, 100, 127, 128, 129, 200, 0]
    say("checkpoints every %d ragged: d=%d %s Hk=%d Hv=%d" % (every, d_head, dtype, hk, hv))
    w = gi.Workload("ragged", 1, 0, hk, hv, d_head, d_head, dtype, seg_range=(1, 2),
                    n_segments=len(lens), seed=93)
    d = gi.generate(w, lengths=lens)
    t = to_device(d)
    rows = (sum(lens) + every - 1) // every + len(lens)
    _check_n(t, d, rows, every, "ckpt/%d ragged d=%d %s" % (every, d_head, dtype))


def test_checkpoints_every_16_fixed_length():
    """Fixed-length rows (B=4, T=512, 16 heads), a checkpoint every 16 tokens:
    32 rows per sequence, three of every four inside a chunk."""
    say("checkpoints every 16, fixed B=4 T=512")
    d = gi.generate(gi.WORKLOADS["fixed_B4_T512_H16_d128"])
    t = to_device(d)
    _check_n(t, d, 4 * 32, 16, "ckpt/16 fixed B4 T512")


def test_checkpoints_n64_equals_chunk_entry_point():
    """every_n = 64 through gdr_chunk_fwd_checkpoints_n gives the rows of
    gdr_chunk_fwd_checkpoints bit for bit; n = 16 rows 3, 7, 11, ... are the
    64-token rows (the chunk-end path) and also equal them bit for bit."""
    import ctypes
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    lens = [300, 0, 64, 129]
    w = gi.Workload("ragged", 1, 0, 2, 4, 128, 128, "bf16", seg_range=(1, 2), n_segments=len(lens), seed=95)
    d = gi.generate(w, lengths=lens)
    t = to_device(d)
    say("checkpoints n=64 via the _n entry point")
    rows = (sum(lens) + 63) // 64 + len(lens)
    _, _, h64 = _run(t, d, rows)
    lib = gdr.library()
    hn = torch.full_like(h64, 7.0)
    o = torch.empty((1, sum(lens), 4, 128), dtype=torch.bfloat16, device="cuda")
    ht = torch.zeros((len(lens), 4, 128, 128), device="cuda")
    ds = [gdr._desc(x) for x in (t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["h0"], o, ht, hn)]
    rc = lib.gdr_chunk_fwd_checkpoints_n(*[gdr._ref(x) for x in ds], ctypes.c_int64(64),
                                         ctypes.c_float(d["scale"]), None)
    torch.cuda.synchronize()
    assert rc == 0, lib.gdr_last_error()
    assert torch.equal(hn, h64)
    # every 16: rows at multiples of 64 come from the same chunk-end stores
    r16 = (sum(lens) + 15) // 16 + len(lens)
    _, _, h16 = _run_n(t, d, r16, 16)
    off16, off64 = 0, 0
    for L in lens:
        n16, n64 = (L + 15) // 16, (L + 63) // 64
        for j in range(n64):
            j16 = min(4 * (j + 1), n16) - 1
            assert torch.equal(h16[off16 + j16], h64[off64 + j]), "L=%d chunk %d" % (L, j)
        off16 += n16
        off64 += n64


@pytest.mark.parametrize("every,dk,dv,dtype", [(16, 128, 64, "bf16"), (64, 64, 128, "bf16"), (32, 128, 64, "fp32")])
def test_checkpoints_independent_head_dims(every, dk, dv, dtype):
    """Checkpoints with dk != dv: rows of [dk][dv] states."""
    lens = [17, 0, 64, 130, 200]
    say("checkpoints every %d, dk=%d dv=%d %s" % (every, dk, dv, dtype))
    w = gi.Workload("ragged", 1, 0, 2, 4, dk, dv, dtype, seg_range=(1, 2), n_segments=len(lens), seed=97)
    d = gi.generate(w, lengths=lens)
    t = to_device(d)
    rows = (sum(lens) + every - 1) // every + len(lens)
    _check_n(t, d, rows, every, "ckpt/%d dk=%d dv=%d %s" % (every, dk, dv, dtype))
