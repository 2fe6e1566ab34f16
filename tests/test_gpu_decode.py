"""GPU: the single-token decode step (gdr_decode_step) against the oracle.

One decode step is one token of the recurrence, so the oracle is its plain
per-token fp64 forward with T = 1 and h0 = the state.  A chain of steps is
checked against the oracle over the same tokens.  Tolerances: o 2e-3 and the
state 2e-2, absolute, as for the forward pass.
"""
import numpy as np
import pytest

import gdr_inputs as gi
from gpu_helpers import TOL_HT, TOL_O, dev, np64, say

pytestmark = pytest.mark.gpu


def _case(seed, B, T, hk, hv, d, dtype, dv=None):
    dv = dv or d
    w = gi.Workload("decode", B, T, hk, hv, d, dv, dtype, seed=seed)
    c = gi.generate(w)
    rng = np.random.default_rng(seed)
    c["h0"] = (0.3 * rng.standard_normal((B, hv, d, dv))).astype(np.float32)
    return c


def _oracle(c):
    import oracle
    return oracle.gdr_fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], None, c["h0"], scale=c["scale"])


def _steps(c, gate_dtype=None):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    dt = c["dtype"]
    gd = gate_dtype or dt
    h = torch.from_numpy(c["h0"]).cuda()
    outs = []
    T = c["q"].shape[1]
    for t in range(T):
        o = gdr.decode_step(dev(c["q"][:, t], dt), dev(c["k"][:, t], dt), dev(c["v"][:, t], dt),
                            dev(c["g"][:, t], gd), dev(c["beta"][:, t], gd), h, scale=c["scale"])
        outs.append(np64(o))
    torch.cuda.synchronize()
    return np.stack(outs, axis=1), np64(h)


@pytest.mark.parametrize("B,hk,hv,d,dtype", [(5, 2, 4, 128, "bf16"), (3, 1, 2, 64, "fp32"),
                                             (64, 16, 32, 128, "bf16"), (2, 2, 2, 128, "fp32")])
def test_decode_one_step(B, hk, hv, d, dtype):
    c = _case(11 + B, B, 1, hk, hv, d, dtype)
    o, h = _steps(c)
    o_ref, h_ref = _oracle(c)
    do = float(np.abs(o - o_ref).max())
    dh = float(np.abs(h - h_ref).max())
    say("decode B=%d Hk=%d Hv=%d d=%d %s: max|do| %.3e max|dh| %.3e" % (B, hk, hv, d, dtype, do, dh))
    assert do <= TOL_O and dh <= TOL_HT


@pytest.mark.parametrize("dk,dv,dtype", [(128, 64, "bf16"), (64, 128, "fp32")])
def test_decode_independent_head_dims(dk, dv, dtype):
    """dk != dv: a chain of 10 steps against the oracle over the same tokens."""
    c = _case(31, 4, 10, 2, 4, dk, dtype, dv=dv)
    o, h = _steps(c)
    o_ref, h_ref = _oracle(c)
    do = float(np.abs(o - o_ref).max())
    dh = float(np.abs(h - h_ref).max())
    say("decode dk=%d dv=%d %s: max|do| %.3e max|dh| %.3e" % (dk, dv, dtype, do, dh))
    assert o.shape == o_ref.shape and do <= TOL_O and dh <= TOL_HT


def test_decode_chain_of_steps():
    c = _case(5, 3, 70, 2, 4, 128, "bf16")
    o, h = _steps(c)
    o_ref, h_ref = _oracle(c)
    do = float(np.abs(o - o_ref).max())
    dh = float(np.abs(h - h_ref).max())
    say("decode chain of 70 steps: max|do| %.3e max|dh| %.3e" % (do, dh))
    assert do <= TOL_O and dh <= TOL_HT


def test_decode_gate_dtype_mix():
    c = _case(9, 4, 2, 2, 2, 64, "bf16")
    c["g"] = gi.round_to_bf16(c["g"]).astype(np.float32)
    o, h = _steps(c, gate_dtype="fp32")
    o_ref, h_ref = _oracle(c)
    assert float(np.abs(o - o_ref).max()) <= TOL_O
    assert float(np.abs(h - h_ref).max()) <= TOL_HT
