"""Backward pass on the GPU against the fp64 backward oracle, element by
element: every gradient (dq, dk, dv, dg, dbeta, dh0) on the seeded workloads,
ragged chunks, ghosts, GQA, both head sizes and both gate dtypes, and the
long and benchmark workloads at full size on every head.
Also: repeated calls and ghost padding are bitwise reproducible."""
import numpy as np
import pytest

from gpu_helpers import dev, np64, say, to_device

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
# max |gpu - oracle| <= TOL[name] * max(1, max |oracle|), per gradient
TOL = dict(dq=1.5e-2, dk=1.5e-2, dv=1.5e-2, dg=1.5e-2, dbeta=1.5e-2, dh0=1.5e-2)


def _case(name, seed=None, lengths=None, gate_dtype=None):
    import gdr_inputs
    w = gdr_inputs.WORKLOADS[name] if isinstance(name, str) else name
    d = gdr_inputs.generate(w, seed=seed, lengths=lengths)
    d.update(gdr_inputs.generate_grads(d, seed=(w.seed if seed is None else seed) + 7))
    return d


def _gpu(d, gate_dtype=None, with_dht=True, h0="same", cu="same"):
    import chunked_gated_delta_fwd_amd as gdr
    import torch
    t = to_device(d, gate_dtype)
    do = dev(d["do"], d["dtype"])
    dht = dev(d["dht"], "fp32") if with_dht else None
    h0_ = t["h0"] if isinstance(h0, str) else h0
    cu_ = t["cu"] if isinstance(cu, str) else cu
    out = gdr.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do, cu_, h0_, dht, scale=d["scale"])
    torch.cuda.synchronize()
    return dict(zip(GRADS, out))


def _oracle(d, with_dht=True, heads=None):
    import oracle
    q, k, v, g, beta, do = d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"]
    h0, dht = d["h0"], d["dht"] if with_dht else None
    if heads is not None:   # (k-heads, v-heads) slice; the v-heads must be exactly those of the k-heads
        kh, vh = heads
        q, k = q[:, :, kh], k[:, :, kh]
        v, g, beta, do = v[:, :, vh], g[:, :, vh], beta[:, :, vh], do[:, :, vh]
        h0 = None if h0 is None else h0[:, vh]
        dht = None if dht is None else dht[:, vh]
    return oracle.gdr_bwd(q, k, v, g, beta, do, cu_seqlens=d["cu_seqlens"], h0=h0, dht=dht, scale=d["scale"])


def _compare(got, ref, what, heads=None, tol=TOL):
    errs = {}
    for n in GRADS:
        if got[n] is None:
            continue
        x = np64(got[n])
        if heads is not None:
            kh, vh = heads
            x = x[:, :, kh] if n in ("dq", "dk") else x[:, vh] if n == "dh0" else x[:, :, vh]
        r = ref[n]
        assert x.shape == r.shape, "%s %s: shape %s vs %s" % (what, n, x.shape, r.shape)
        assert np.all(np.isfinite(x)), "%s: non-finite %s" % (what, n)
        err = float(np.abs(x - r).max()) if r.size else 0.0
        mag = max(1.0, float(np.abs(r).max())) if r.size else 1.0
        errs[n] = err / mag
    say("%s: " % what + "  ".join("%s %.2e" % (n, e) for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol[n], "%s: %s error %.3e > %.1e (relative to max(1, max|ref|))" % (what, n, e, tol[n])
    return errs


@pytest.mark.parametrize("name", ["tiny_fp32_T128_H2_d64", "fixed_B4_T512_H16_d128", "varlen8_ghost8_H32_d128"])
def test_bwd_workloads(name):
    d = _case(name)
    _compare(_gpu(d), _oracle(d), name)


def test_bwd_gqa_ragged_ghosts_d128():
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(31, n_real=6, lo=1, hi=300, ghost_slots=4, hk=2, hv=8, d=128)
    d.update(gdr_inputs.generate_grads(d, seed=32))
    _compare(_gpu(d), _oracle(d), "gqa4 ragged ghosts d128")


def test_bwd_gqa_d64_fp32_gates_no_state():
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(41, n_real=4, lo=30, hi=200, ghost_slots=2, hk=1, hv=4, d=64,
                                       with_h0=False)
    d.update(gdr_inputs.generate_grads(d, seed=42))
    _compare(_gpu(d, gate_dtype="fp32", with_dht=False), _oracle(d, with_dht=False),
             "gqa4 d64 fp32 gates, no h0, no dht")


def test_bwd_gqa_d64_with_state():
    """d = 64 with h0 (the first chunk of each segment stages h0, the others the
    recomputed chunk states) and dht, GQA, ragged segments and ghosts."""
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(43, n_real=4, lo=30, hi=260, ghost_slots=2, hk=2, hv=4, d=64)
    d.update(gdr_inputs.generate_grads(d, seed=44))
    _compare(_gpu(d), _oracle(d), "gqa d64 with h0 and dht")


def test_bwd_gqa_odd_group_d128():
    """Three v-heads per q/k head: the prep kernel then takes one v-head per
    work-group (it pairs v-heads only within a q/k head)."""
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(61, n_real=3, lo=20, hi=180, ghost_slots=1, hk=2, hv=6, d=128)
    d.update(gdr_inputs.generate_grads(d, seed=62))
    _compare(_gpu(d), _oracle(d), "gqa3 d128")


def test_bwd_fp32_inputs_d128():
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(51, n_real=3, lo=60, hi=200, ghost_slots=1, hk=2, hv=2, d=128,
                                       dtype="fp32")
    d.update(gdr_inputs.generate_grads(d, seed=52))
    _compare(_gpu(d), _oracle(d), "fp32 inputs d128")


@pytest.mark.parametrize("g_mode", ["logsigmoid/16", "zero"])
def test_bwd_slow_and_no_decay(g_mode):
    """Gates that decay slowly or not at all, so the state gradient carries
    across many chunks (with logsigmoid(N(0, 1)) gates a chunk decays by about
    e^-50 and the chunk-to-chunk recursion barely reaches the other chunks'
    gradients): segments of up to 700 tokens, GQA, ghosts."""
    import gdr_inputs
    w = gdr_inputs.Workload("slow", 1, 0, 2, 4, 128, 128, "bf16", seg_range=(100, 700), n_segments=5,
                            seed=71)
    d = gdr_inputs.generate(w, g_mode=g_mode)
    d.update(gdr_inputs.generate_grads(d, seed=72))
    _compare(_gpu(d), _oracle(d), "decay %s" % g_mode)


def test_bwd_long_all_heads():
    """T = 20468 (last chunk 52 tokens), 16 heads: all gradients of every head."""
    d = _case("long_T20468_H16_d128")
    got = _gpu(d)
    _compare(got, _oracle(d), "long T20468 all heads")


def test_bwd_packed64k_all_heads():
    """The benchmark workload at full size: all six gradients of every head,
    element by element (the fp64 oracle takes about half a minute on 16 cores)."""
    d = _case("packed64k_gqa_Hk16_Hv32_d128")
    got = _gpu(d)
    _compare(got, _oracle(d), "packed64k all heads")


def test_bwd_bitwise_repeatable_and_ghost_padding():
    import torch
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(61, n_real=5, lo=1, hi=260, ghost_slots=0, hk=2, hv=4, d=128)
    d.update(gdr_inputs.generate_grads(d, seed=62))
    a = _gpu(d)
    b = _gpu(d)
    for n in GRADS:
        assert torch.equal(a[n], b[n]), "second call differs in %s" % n
    # the same segments with ghosts appended (their dh0 rows must stay untouched)
    cu = d["cu_seqlens"]
    cu2 = np.concatenate([cu, np.full(5, cu[-1], dtype=cu.dtype)])
    t = to_device(d)
    import chunked_gated_delta_fwd_amd as gdr
    h0 = torch.cat([t["h0"], torch.zeros((5,) + tuple(t["h0"].shape[1:]), device="cuda")])
    dht = torch.cat([dev(d["dht"], "fp32"), torch.ones((5,) + tuple(t["h0"].shape[1:]), device="cuda")])
    sentinel = torch.full((len(cu2) - 1,) + tuple(t["h0"].shape[1:]), 3.5, device="cuda")
    out = gdr.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], dev(d["do"], d["dtype"]),
                        dev(cu2, "i32"), h0, dht, scale=d["scale"], dh0=sentinel)
    torch.cuda.synchronize()
    for n, x in zip(GRADS, out):
        if n == "dh0":
            assert torch.equal(x[:len(cu) - 1], a[n]), "ghost padding changed dh0"
            assert torch.all(x[len(cu) - 1:] == 3.5), "ghost rows of dh0 written"
        else:
            assert torch.equal(x, a[n]), "ghost padding changed %s" % n
