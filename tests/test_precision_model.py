"""Where the forward kernel's error comes from (CPU, a model of its roundings;
see tests/precision_model.py).  With no decay, where the state carries every
rounding across chunks, the diagonal-block inverse's own precision is not what
limits accuracy: an exact inverse leaves the error within a few percent, while
keeping Vnew (the MFMA operand of P Vnew and of the state update) unrounded
roughly halves the state error.  The model also reproduces the GPU's error
scale, so it stays a faithful stand-in."""
import numpy as np
import pytest

import precision_model as pm


@pytest.mark.parametrize("T", [512, 2048])
def test_inverse_precision_is_not_the_limit(T):
    q, k, v, g, b, h0, scale = pm.case(T, "zero")
    o_ref, h_ref = pm.reference(q, k, v, g, b, h0, scale)
    err = {}
    for name, kw in (("kernel", {}), ("exact_inverse", {"exact_inverse": True}),
                     ("fp_vnew", {"round_vnew": False}), ("fp_o", {"round_o": False})):
        o, h = pm.kernel_model(q, k, v, g, b, h0, scale, **kw)
        err[name] = (np.abs(o - o_ref).max(), np.abs(h - h_ref).max())
    do, dh = err["kernel"]
    # the model's error scale matches the GPU's (no decay: 1.2e-3 / 9.2e-3 at T = 512)
    assert 5e-4 < do < 2e-3 and 3e-3 < dh < 2e-2
    # an exact inverse changes the output and state errors by under 15 %
    assert abs(err["exact_inverse"][0] - do) < 0.15 * do
    assert abs(err["exact_inverse"][1] - dh) < 0.15 * dh
    # the Vnew rounding dominates the state error, the output rounding is a
    # large share of the output error
    assert err["fp_vnew"][1] < 0.6 * dh
    assert err["fp_o"][0] < 0.85 * do
