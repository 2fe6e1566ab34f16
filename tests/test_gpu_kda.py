"""Per-channel-gate forward (gdr_chunk_kda_fwd) on the GPU against the fp64
oracle gdr_kda_fwd, element by element, with the forward's tolerances: the
seeded workloads with one log-gate per key channel, ragged chunks, ghosts, GQA,
both head sizes, fp32 gates; the full packed workload on every head.  f32
inputs run in fp32 arithmetic and meet the f32 tolerances, at any gate."""
import numpy as np
import pytest

from gpu_helpers import dev, np64, say, to_device, tols

pytestmark = pytest.mark.gpu


def _run(d, gk, gate_dtype=None):
    import chunked_gated_delta_fwd_amd as gdr
    import torch
    t = to_device(d, gate_dtype)
    g = dev(gk, gate_dtype or d["dtype"])
    o, ht = gdr.chunk_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], t["cu"], t["h0"], scale=d["scale"])
    torch.cuda.synchronize()
    return np64(o), np64(ht)


def _ref(d, gk, heads=None):
    import oracle
    q, k, v, g, beta, h0 = d["q"], d["k"], d["v"], gk, d["beta"], d["h0"]
    if heads is not None:
        kh, vh = heads
        q, k, v, g, beta = q[:, :, kh], k[:, :, kh], v[:, :, vh], g[:, :, vh], beta[:, :, vh]
        h0 = None if h0 is None else h0[:, vh]
    return oracle.gdr_kda_fwd(q, k, v, g, beta, d["cu_seqlens"], h0, scale=d["scale"])


def _check(o, ht, o_ref, ht_ref, real, what, dtype="bf16"):
    tol_o, tol_ht = tols(dtype)
    e_o = float(np.abs(o - o_ref).max())
    e_h = float(np.abs(ht[real] - ht_ref[real]).max()) if len(real) else 0.0
    say("%s: max|do| %.3e (max_ref %.3f)  max|dht| %.3e (max_ref %.3f)"
        % (what, e_o, float(np.abs(o_ref).max()), e_h, float(np.abs(ht_ref).max())))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht)), what + ": non-finite"
    assert e_o <= tol_o, "%s: max|do| %.3e > %.1e" % (what, e_o, tol_o)
    assert e_h <= tol_ht, "%s: max|dht| %.3e > %.1e" % (what, e_h, tol_ht)


def _real(d):
    cu = d["cu_seqlens"]
    if cu is None:
        return list(range(len(d["lengths"])))
    return [i for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]


@pytest.mark.parametrize("name", ["tiny_fp32_T128_H2_d64", "fixed_B4_T512_H16_d128", "varlen8_ghost8_H32_d128"])
def test_kda_workloads(name):
    import gdr_inputs
    w = gdr_inputs.WORKLOADS[name]
    d = gdr_inputs.generate(w)
    gk = gdr_inputs.generate_kda_gates(d, seed=w.seed + 3)
    o, ht = _run(d, gk)
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda " + name, w.dtype)


def test_kda_gqa_ragged_ghosts():
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(81, n_real=6, lo=1, hi=300, ghost_slots=4, hk=2, hv=8, d=128)
    gk = gdr_inputs.generate_kda_gates(d, seed=82)
    o, ht = _run(d, gk)
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda gqa4 ragged ghosts")


def test_kda_d64_fp32_gates_slow_decay():
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(83, n_real=3, lo=100, hi=400, ghost_slots=1, hk=1, hv=2, d=64)
    gk = gdr_inputs.generate_kda_gates(d, seed=84, scale=1.0 / 16)
    o, ht = _run(d, gk, gate_dtype="fp32")
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda d64 fp32 gates, slow decay")


def test_kda_fast_decay():
    """Gates twice as steep (mean about -1.6 per token and channel: half a chunk
    sums to about -51, inside the documented range of about -85)."""
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(85, n_real=3, lo=64, hi=200, ghost_slots=0, hk=2, hv=2, d=128)
    gk = gdr_inputs.generate_kda_gates(d, seed=86, scale=2.0)
    o, ht = _run(d, gk)
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda fast decay")


@pytest.mark.parametrize("mode", ["const-5", "uniform-5..0"])
def test_kda_bf16_gates_at_safe_lower_bound(mode):
    """bf16 inputs with every per-channel log-decay at -5 per token (the pages'
    safe-gate lower bound), or uniform in [-5, 0] per token and channel: the
    16-row block references keep every factor inside fp32, no range flag is
    raised, and o and ht match the oracle at the bf16 tolerances."""
    import chunked_gated_delta_fwd_amd as gdr
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(88, n_real=4, lo=1, hi=300, ghost_slots=1, hk=2, hv=4, d=128)
    shape = d["v"].shape[:3] + (d["q"].shape[3],)
    if mode == "const-5":
        gk = np.full(shape, -5.0, dtype=np.float32)
    else:
        gk = gdr_inputs.round_to_bf16(
            -5.0 * np.random.Generator(np.random.PCG64(89)).random(shape).astype(np.float32))
    say("kda bf16 gates %s" % mode)
    assert gdr.device_status(clear=True) == 0
    o, ht = _run(d, gk)
    assert gdr.device_status() == 0, "range flag raised inside the documented range"
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda bf16 g %s" % mode)


def test_kda_bf16_gates_beyond_range_are_flagged():
    """Gates of -6 per token (-96 over a 16-token block, beyond fp32's
    exponent range) set GDR_DEVSTAT_KDA_RANGE; the next in-range call is clean."""
    import chunked_gated_delta_fwd_amd as gdr
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(90, n_real=2, lo=40, hi=80, ghost_slots=0, hk=1, hv=2, d=64)
    shape = d["v"].shape[:3] + (d["q"].shape[3],)
    say("kda bf16 gates -6: range flag")
    assert gdr.device_status(clear=True) == 0
    _run(d, np.full(shape, -6.0, dtype=np.float32))
    bits = gdr.device_status(clear=True)
    assert bits & gdr.GDR_DEVSTAT_KDA_RANGE, bits
    gk = np.full(shape, -1.0, dtype=np.float32)
    o, ht = _run(d, gk)
    assert gdr.device_status() == 0
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda bf16 g -1 after a flagged call")


@pytest.mark.parametrize("gval", [-5.0, -60.0])
def test_kda_f32_inputs_steep_gates(gval):
    """f32 inputs with every per-channel log-decay at gval per token (half a
    chunk sums to -160 or -1920, far outside the bf16 kernel's range): the fp32
    kernel applies each token's decay directly, so any gate is in range."""
    import gdr_inputs
    d = gdr_inputs.random_lengths_case(87, n_real=3, lo=1, hi=200, ghost_slots=1, hk=1, hv=2, d=128,
                                       dtype="fp32")
    gk = np.full(d["v"].shape[:3] + (d["q"].shape[3],), gval, dtype=np.float32)
    say("kda f32 inputs, g = %g per token and channel" % gval)
    o, ht = _run(d, gk)
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda f32 g=%g" % gval, "fp32")


def test_kda_packed64k_all_heads():
    """The benchmark workload with per-channel gates, every head element by
    element (the fp64 oracle takes about ten seconds on 16 cores)."""
    import gdr_inputs
    w = gdr_inputs.WORKLOADS["packed64k_gqa_Hk16_Hv32_d128"]
    d = gdr_inputs.generate(w)
    gk = gdr_inputs.generate_kda_gates(d, seed=w.seed + 3)
    o, ht = _run(d, gk)
    o_ref, ht_ref = _ref(d, gk)
    _check(o, ht, o_ref, ht_ref, _real(d), "kda packed64k all heads")
