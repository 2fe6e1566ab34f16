"""Shared helpers of the GPU tests: move seeded inputs to the device, call the
HIP path through the C ABI, call the oracle on the same values, compare."""
from __future__ import annotations

import sys

import numpy as np

TOL_O = 2e-3    # max |o_gpu - o_oracle|, absolute (bf16 inputs: bf16 MFMA operands)
TOL_HT = 2e-2   # max |ht_gpu - ht_oracle|, absolute
# f32 inputs run in fp32 arithmetic throughout: the worst case measured, 20468
# tokens with no decay, stays within 1.3e-7 (o) and 1.5e-6 (state) of the oracle
TOL_O_F32 = 2e-6
TOL_HT_F32 = 2e-5


def tols(dtype: str):
    """(tolerance of o, tolerance of ht) for inputs of `dtype`."""
    return (TOL_O_F32, TOL_HT_F32) if dtype == "fp32" else (TOL_O, TOL_HT)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype: str):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if t.dtype == torch.int32 or t.dtype == torch.int64:
        return t.to(torch.int32).cuda()
    t = t.to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def to_device(d: dict, gate_dtype: str = None):
    """Device tensors of a generated case (q/k/v/g/beta in the case's dtype)."""
    dt = d["dtype"]
    gd = gate_dtype or dt
    return dict(q=dev(d["q"], dt), k=dev(d["k"], dt), v=dev(d["v"], dt), g=dev(d["g"], gd),
                beta=dev(d["beta"], gd), cu=dev(d["cu_seqlens"], "i32"),
                h0=None if d["h0"] is None else dev(d["h0"], "fp32"))


def run_gpu(t: dict, scale: float, ht_init=None, cu="same", h0="same"):
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    cu_ = t["cu"] if isinstance(cu, str) else cu
    h0_ = t["h0"] if isinstance(h0, str) else h0
    N = (cu_.shape[0] - 1) if cu_ is not None else t["q"].shape[0]
    ht = None
    if ht_init is not None:
        ht = ht_init.clone()
    else:
        ht = torch.zeros((N,) + tuple(t["v"].shape[2:3]) + (t["q"].shape[3], t["v"].shape[3]),
                         dtype=torch.float32, device="cuda")
    o, ht = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_, h0_, scale=scale, ht=ht)
    torch.cuda.synchronize()
    return o, ht


def np64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def run_oracle(d: dict, cu="same", h0="same", ht_init=None):
    import oracle
    cu_ = d["cu_seqlens"] if isinstance(cu, str) else cu
    h0_ = d["h0"] if isinstance(h0, str) else h0
    return oracle.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_, h0_, scale=d["scale"],
                          ht_init=ht_init)


def compare(o_gpu, ht_gpu, o_ref, ht_ref, what: str, tol_o=TOL_O, tol_ht=TOL_HT, rows=None):
    """Element-wise comparison over every element (or the given o rows)."""
    o = np64(o_gpu) if not isinstance(o_gpu, np.ndarray) else o_gpu
    ht = np64(ht_gpu) if not isinstance(ht_gpu, np.ndarray) else ht_gpu
    if rows is not None:
        o, o_ref = o[rows], o_ref[rows]
    assert np.all(np.isfinite(o)), "%s: non-finite o" % what
    assert np.all(np.isfinite(ht)), "%s: non-finite ht" % what
    do = float(np.abs(o - o_ref).max()) if o.size else 0.0
    dh = float(np.abs(ht - ht_ref).max()) if ht.size else 0.0
    mref_o = float(np.abs(o_ref).max()) if o.size else 0.0
    mref_h = float(np.abs(ht_ref).max()) if ht.size else 0.0
    cos = float(np.sum(o * o_ref) / max(1e-300, np.linalg.norm(o) * np.linalg.norm(o_ref))) if o.size else 1.0
    say("%s: max|do| %.3e (max_ref %.4f, mean %.2e, cos %.6f)  max|dht| %.3e (max_ref %.4f)"
        % (what, do, mref_o, float(np.abs(o - o_ref).mean()) if o.size else 0.0, cos, dh, mref_h))
    assert do <= tol_o, "%s: max|do| %.3e > %.1e" % (what, do, tol_o)
    assert dh <= tol_ht, "%s: max|dht| %.3e > %.1e" % (what, dh, tol_ht)
    return do, dh
