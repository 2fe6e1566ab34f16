"""Chunked gated delta rule forward for AMD MI355X (gfx950).

A thin ctypes binding over ``libgdr.so`` (HIP kernels behind the C ABI of
``include/gdr.h``).  Every step of the computation runs in the library's
kernels; this module only marshals torch tensors into descriptors and passes
torch's current HIP stream.  There is no fallback: if the library is missing
or the device is not gfx950, calls raise.

The op is ``chunk_gated_delta_rule`` (chunk size 64, varlen ``cu_seqlens``,
initial/final state) as named on the FlashQLA pages; per sequence and v-head
``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T`` and
``o_t = scale S_t q_t``, the state returned as ``H = S^T`` ``[N, Hv, dk, dv]``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_F32, GDR_BF16, GDR_I32 = 0, 1, 2
STATUS = {0: "GDR_OK", -1: "GDR_EINVAL", -2: "GDR_ESHAPE", -3: "GDR_EDTYPE", -4: "GDR_ESTRIDE",
          -5: "GDR_EALIAS", -6: "GDR_EDEVICE", -7: "GDR_ELAUNCH", -8: "GDR_ENOMEM"}

# every symbol include/gdr.h declares
EXPORTS = ("gdr_chunk_fwd", "gdr_chunk_fwd_checkpoints", "gdr_chunk_bwd", "gdr_chunk_kda_fwd", "gdr_decode_step", "gdr_plan",
           "gdr_prepare_chunks", "gdr_dispatch_order",
           "gdr_chunk_local_cumsum", "gdr_last_error", "gdr_version", "gdr_selftest_mfma",
           "gdr_debug_set", "gdr_device_status", "gdr_free_workspaces", "gdr_chunk_fwd_noalloc",
           "gdr_chunk_fwd_checkpoints_n")

# gdr_debug_set options and device status bits (include/gdr.h)
GDR_DEBUG_CHECK_CU, GDR_DEBUG_FAIL_LAUNCHES, GDR_DEBUG_SPIN_LIMIT = 1, 2, 3
GDR_DEVSTAT_WAIT_TIMEOUT = 1
GDR_DEVSTAT_KDA_RANGE = 2


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, message))
        self.status = status
        self.message = message


class GdrTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.POINTER(ctypes.c_int64)), ("strides", ctypes.POINTER(ctypes.c_int64))]


class GdrLaunchPlan(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int64), ("total_tokens", ctypes.c_int64), ("nt_max", ctypes.c_int64),
                ("hk", ctypes.c_int32), ("hv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32), ("varlen", ctypes.c_int32),
                ("has_h0", ctypes.c_int32), ("has_ht", ctypes.c_int32), ("grid_fwd", ctypes.c_int64),
                ("block_fwd", ctypes.c_int32), ("lds_fwd", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("dv", ctypes.c_int32)]


_lib = None


def library(path: Optional[str] = None):
    """Load ``libgdr.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libgdr.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    TP = ctypes.POINTER(GdrTensor)
    lib.gdr_chunk_fwd.argtypes = [TP] * 9 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd_noalloc.argtypes = [TP] * 9 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_fwd_checkpoints.argtypes = [TP] * 10 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_fwd_checkpoints.restype = ctypes.c_int
    lib.gdr_chunk_fwd_checkpoints_n.argtypes = [TP] * 10 + [ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_fwd_checkpoints_n.restype = ctypes.c_int
    lib.gdr_chunk_kda_fwd.argtypes = [TP] * 9 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_kda_fwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [TP] * 15 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_decode_step.argtypes = [TP] * 7 + [ctypes.c_float, ctypes.c_void_p]
    lib.gdr_decode_step.restype = ctypes.c_int
    lib.gdr_plan.argtypes = [TP] * 9 + [ctypes.c_float, ctypes.POINTER(GdrLaunchPlan)]
    lib.gdr_plan.restype = ctypes.c_int
    lib.gdr_prepare_chunks.argtypes = [TP] * 4 + [ctypes.c_void_p]
    lib.gdr_prepare_chunks.restype = ctypes.c_int
    lib.gdr_dispatch_order.argtypes = [TP, ctypes.c_int32, TP, ctypes.c_void_p]
    lib.gdr_dispatch_order.restype = ctypes.c_int
    lib.gdr_chunk_local_cumsum.argtypes = [TP] * 3 + [ctypes.c_void_p]
    lib.gdr_chunk_local_cumsum.restype = ctypes.c_int
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = ctypes.c_int
    lib.gdr_selftest_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.gdr_selftest_mfma.restype = ctypes.c_int
    lib.gdr_debug_set.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.gdr_debug_set.restype = ctypes.c_int
    lib.gdr_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    lib.gdr_device_status.restype = ctypes.c_int
    lib.gdr_free_workspaces.argtypes = []
    lib.gdr_free_workspaces.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(lib, status: int):
    if status != 0:
        raise GdrError(status, lib.gdr_last_error().decode("utf-8", "replace"))


class _Desc:
    """A gdr_tensor plus the shape/stride arrays it points to."""

    def __init__(self, data: int, dtype: int, shape: Sequence[int], strides: Optional[Sequence[int]]):
        n = len(shape)
        self._shape = (ctypes.c_int64 * max(n, 1))(*shape)
        self._strides = None if strides is None else (ctypes.c_int64 * max(n, 1))(*strides)
        self.t = GdrTensor(ctypes.c_void_p(data), dtype, n,
                           ctypes.cast(self._shape, ctypes.POINTER(ctypes.c_int64)),
                           None if self._strides is None else
                           ctypes.cast(self._strides, ctypes.POINTER(ctypes.c_int64)))

    @property
    def ref(self):
        return ctypes.byref(self.t)


def describe(data: int, dtype: int, shape: Sequence[int], strides: Optional[Sequence[int]] = None) -> _Desc:
    """Descriptor from a raw address (used by host-only planning tests)."""
    return _Desc(int(data), int(dtype), [int(s) for s in shape],
                 None if strides is None else [int(s) for s in strides])


def _torch_dtype_code(t) -> int:
    import torch
    m = {torch.float32: GDR_F32, torch.bfloat16: GDR_BF16, torch.int32: GDR_I32}
    if t.dtype not in m:
        raise GdrError(-3, "unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _desc(t) -> Optional[_Desc]:
    if t is None:
        return None
    return _Desc(t.data_ptr(), _torch_dtype_code(t), list(t.shape), list(t.stride()))


def _ref(d: Optional[_Desc]):
    return None if d is None else d.ref


def _stream_handle(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def chunk_fwd(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None,
              output_final_state: bool = True, o=None, ht=None) -> Tuple[object, Optional[object]]:
    """Forward of chunk_gated_delta_rule on torch tensors (device memory).

    q, k ``[B,T,Hk,d]``; v ``[B,T,Hv,d]``; g, beta ``[B,T,Hv]``; ``cu_seqlens``
    int32 ``[N+1]`` (B == 1) or None; h0 f32 ``[N,Hv,d,d]`` or None.  Returns
    ``(o, ht)``; ``ht`` is None unless ``output_final_state``.  ``o``/``ht`` may be
    given preallocated (ghost rows of ``ht`` keep their contents).
    """
    import torch
    lib = library()
    B, T, Hk, d = q.shape
    Hv = v.shape[2]
    N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else B
    if scale is None:
        scale = float(d) ** -0.5
    if o is None:
        o = torch.empty((B, T, Hv, v.shape[3]), dtype=q.dtype, device=q.device)
    if ht is None and output_final_state:
        ht = torch.zeros((N, Hv, d, v.shape[3]), dtype=torch.float32, device=q.device)
    ds = [_desc(x) for x in (q, k, v, g, beta, cu_seqlens, h0, o, ht)]
    _check(lib, lib.gdr_chunk_fwd(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                  ctypes.c_void_p(_stream_handle(q))))
    return o, ht


def chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None, o=None, ht=None):
    """``chunk_fwd`` through the entry point that allocates no device memory
    (its workspace is a static device array shared by every call on the GPU).
    ``o`` and ``ht`` are allocated here when not given; pass them preallocated
    when this runs where allocation is not allowed."""
    import torch
    lib = library()
    B, T, Hk, d = q.shape
    Hv = v.shape[2]
    N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else B
    if scale is None:
        scale = float(d) ** -0.5
    if o is None:
        o = torch.empty((B, T, Hv, v.shape[3]), dtype=q.dtype, device=q.device)
    if ht is None:
        ht = torch.zeros((N, Hv, d, v.shape[3]), dtype=torch.float32, device=q.device)
    ds = [_desc(x) for x in (q, k, v, g, beta, cu_seqlens, h0, o, ht)]
    _check(lib, lib.gdr_chunk_fwd_noalloc(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                          ctypes.c_void_p(_stream_handle(q))))
    return o, ht


def chunk_fwd_checkpoints(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None,
                          o=None, ht=None, h_chunks=None, every_n: int = 64):
    """``chunk_fwd`` that also returns the state after every 64-token chunk:
    ``(o, ht, h_chunks)`` with h_chunks fp32 ``[R, Hv, dk, dv]``, R = ceil(T/64) + N
    with ``cu_seqlens`` (rows past the true chunk count are not written) or
    B * ceil(T/64); chunk c of sequence n at row sum(ceil(L_m/64), m < n) + c.
    ``every_n`` (a multiple of 16) replaces 64 by that many tokens
    (gdr_chunk_fwd_checkpoints_n; 64 calls gdr_chunk_fwd_checkpoints)."""
    import torch
    lib = library()
    B, T, Hk, d = q.shape
    Hv = v.shape[2]
    N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else B
    if scale is None:
        scale = float(d) ** -0.5
    n = int(every_n)
    rows = ((T + n - 1) // n + N) if cu_seqlens is not None else B * ((T + n - 1) // n)
    if o is None:
        o = torch.empty((B, T, Hv, v.shape[3]), dtype=q.dtype, device=q.device)
    if ht is None:
        ht = torch.zeros((N, Hv, d, v.shape[3]), dtype=torch.float32, device=q.device)
    if h_chunks is None:
        h_chunks = torch.zeros((rows, Hv, d, v.shape[3]), dtype=torch.float32, device=q.device)
    ds = [_desc(x) for x in (q, k, v, g, beta, cu_seqlens, h0, o, ht, h_chunks)]
    if n == 64:
        _check(lib, lib.gdr_chunk_fwd_checkpoints(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                                  ctypes.c_void_p(_stream_handle(q))))
    else:
        _check(lib, lib.gdr_chunk_fwd_checkpoints_n(*[_ref(x) for x in ds], ctypes.c_int64(n),
                                                    ctypes.c_float(scale), ctypes.c_void_p(_stream_handle(q))))
    return o, ht, h_chunks


def chunk_kda_fwd(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None, o=None, ht=None):
    """``chunk_fwd`` with per-channel gates: g ``[B, T, Hv, dk]`` (log-decay of
    each key channel), beta ``[B, T, Hv]``.  Returns ``(o, ht)``."""
    import torch
    lib = library()
    B, T, Hk, d = q.shape
    Hv = v.shape[2]
    N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else B
    if scale is None:
        scale = float(d) ** -0.5
    if o is None:
        o = torch.zeros((B, T, Hv, v.shape[3]), dtype=q.dtype, device=q.device)
    if ht is None:
        ht = torch.zeros((N, Hv, d, v.shape[3]), dtype=torch.float32, device=q.device)
    ds = [_desc(x) for x in (q, k, v, g, beta, cu_seqlens, h0, o, ht)]
    _check(lib, lib.gdr_chunk_kda_fwd(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                      ctypes.c_void_p(_stream_handle(q))))
    return o, ht


def chunk_bwd(q, k, v, g, beta, do, cu_seqlens=None, h0=None, dht=None, scale: Optional[float] = None,
              dq=None, dk=None, dv=None, dg=None, dbeta=None, dh0=None, want_dh0: bool = True):
    """Backward pass of ``chunk_fwd``: given ``do`` ``[B, T, Hv, dv]`` (dtype of
    q) and ``dht`` fp32 ``[N, Hv, dk, dv]`` (or None), returns
    ``(dq, dk, dv, dg, dbeta, dh0)``: dq, dk ``[B, T, Hk, dk]`` and dv in q's
    dtype, dg and dbeta fp32 ``[B, T, Hv]``, dh0 fp32 ``[N, Hv, dk, dv]`` (None
    when ``want_dh0`` is False).  Outputs not given are allocated zeroed (rows
    of tokens outside every segment are not written)."""
    import torch
    lib = library()
    B, T, Hk, d = q.shape
    Hv = v.shape[2]
    N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else B
    if scale is None:
        scale = float(d) ** -0.5
    dev = q.device
    if dq is None:
        dq = torch.zeros_like(q)
    if dk is None:
        dk = torch.zeros_like(k)
    if dv is None:
        dv = torch.zeros_like(v)
    if dg is None:
        dg = torch.zeros((B, T, Hv), dtype=torch.float32, device=dev)
    if dbeta is None:
        dbeta = torch.zeros((B, T, Hv), dtype=torch.float32, device=dev)
    if dh0 is None and want_dh0:
        dh0 = torch.zeros((N, Hv, d, v.shape[3]), dtype=torch.float32, device=dev)
    ds = [_desc(x) for x in (q, k, v, g, beta, cu_seqlens, h0, do, dht, dq, dk, dv, dg, dbeta, dh0)]
    _check(lib, lib.gdr_chunk_bwd(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                  ctypes.c_void_p(_stream_handle(q))))
    return dq, dk, dv, dg, dbeta, dh0


def decode_step(q, k, v, g, beta, h, scale: Optional[float] = None, o=None):
    """One recurrent step per sequence: q, k ``[B, Hk, dk]``, v ``[B, Hv, dv]``,
    g, beta ``[B, Hv]``, state h fp32 ``[B, Hv, dk, dv]`` updated in place.
    Returns o ``[B, Hv, dv]``."""
    import torch
    lib = library()
    B, Hk, d = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if scale is None:
        scale = float(d) ** -0.5
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    ds = [_desc(x) for x in (q, k, v, g, beta, h, o)]
    _check(lib, lib.gdr_decode_step(*[_ref(x) for x in ds], ctypes.c_float(scale),
                                    ctypes.c_void_p(_stream_handle(q))))
    return o


def plan(q, k, v, g, beta, cu_seqlens=None, h0=None, o=None, ht=None, scale: float = 1.0) -> dict:
    """The launch plan for these descriptors (no device access)."""
    lib = library()
    p = GdrLaunchPlan()
    ds = [x if (x is None or isinstance(x, _Desc)) else _desc(x)
          for x in (q, k, v, g, beta, cu_seqlens, h0, o, ht)]
    _check(lib, lib.gdr_plan(*[_ref(x) for x in ds], ctypes.c_float(scale), ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in GdrLaunchPlan._fields_}


def prepare_chunks(cu_seqlens, nt_max: Optional[int] = None, with_map: bool = True,
                   with_order: bool = True):
    """Chunk offsets [N+1], chunk map [nt_max, 2] and longest-first order [N]
    derived on the device from the content of ``cu_seqlens``."""
    import torch
    lib = library()
    N = cu_seqlens.shape[0] - 1
    dev = cu_seqlens.device
    offs = torch.empty(N + 1, dtype=torch.int32, device=dev)
    if nt_max is None:
        nt_max = 0
    cmap = torch.empty((nt_max, 2), dtype=torch.int32, device=dev) if with_map else None
    order = torch.empty(N, dtype=torch.int32, device=dev) if with_order else None
    ds = [_desc(x) for x in (cu_seqlens, offs, cmap, order)]
    _check(lib, lib.gdr_prepare_chunks(*[_ref(x) for x in ds], ctypes.c_void_p(_stream_handle(cu_seqlens))))
    return offs, cmap, order


def dispatch_order(cu_seqlens, groups: int):
    """The order [N] in which the forward pass starts the sequences, for a
    schedule of ``groups`` machines (see ``gdr_dispatch_order``)."""
    import torch
    lib = library()
    N = cu_seqlens.shape[0] - 1
    order = torch.empty(max(N, 0), dtype=torch.int32, device=cu_seqlens.device)
    ds = [_desc(x) for x in (cu_seqlens, order)]
    _check(lib, lib.gdr_dispatch_order(_ref(ds[0]), ctypes.c_int32(groups), _ref(ds[1]),
                                       ctypes.c_void_p(_stream_handle(cu_seqlens))))
    return order


def chunk_local_cumsum(g, cu_seqlens=None, out=None):
    """Chunk-local (64-token) inclusive prefix sum of the log-gate, fp32."""
    import torch
    lib = library()
    if out is None:
        out = torch.zeros(g.shape, dtype=torch.float32, device=g.device)
    ds = [_desc(x) for x in (g, cu_seqlens, out)]
    _check(lib, lib.gdr_chunk_local_cumsum(*[_ref(x) for x in ds], ctypes.c_void_p(_stream_handle(g))))
    return out


def selftest_mfma(a_bits, b_bits):
    """Run the MFMA layout self-test on int16 device tensors of 64x8 bf16 bits."""
    import torch
    lib = library()
    c = torch.zeros(512, dtype=torch.float32, device=a_bits.device)
    _check(lib, lib.gdr_selftest_mfma(ctypes.c_void_p(a_bits.data_ptr()), ctypes.c_void_p(b_bits.data_ptr()),
                                      ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(_stream_handle(a_bits))))
    return c


def debug_set(option: int, value: int) -> None:
    """Process-wide debug / test option (``GDR_DEBUG_*``), see include/gdr.h."""
    lib = library()
    _check(lib, lib.gdr_debug_set(int(option), int(value)))


def device_status(clear: bool = False) -> int:
    """Sticky status bits the kernels set on the current device
    (``GDR_DEVSTAT_*``); synchronises the device."""
    lib = library()
    bits = ctypes.c_uint32(0)
    _check(lib, lib.gdr_device_status(ctypes.byref(bits), 1 if clear else 0))
    return int(bits.value)


def free_workspaces() -> None:
    """Release the current device's library workspaces."""
    lib = library()
    _check(lib, lib.gdr_free_workspaces())


def version() -> int:
    return library().gdr_version()
