"""Oracle for the gated delta rule forward pass — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path never does, and
this package imports nothing from it: the two share no code.

``gdr_fwd`` is a plain per-token fp64 recurrence written in C
(``gdr_oracle.c``) and driven through ctypes over NumPy arrays.  The op is
``chunk_gated_delta_rule`` as named on the FlashQLA pages ("FlashQLA GDN
backend produces different tokens from FLA Triton", Setup: chunk size 64,
varlen API, initial and final state).  The pages do not write the formula;
the recurrence is the gated delta rule of Gated DeltaNet,
``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T`` and
``o_t = scale * S_t q_t``, with the state kept as ``H = S^T`` in
``[N, Hv, dk, dv]`` layout.

``gdr_kda_fwd`` is the same recurrence with one log-gate per key channel
(decay ``diag(exp(g_t))`` on the rows of H), the KDA-style variant.

``gdr_bwd`` is the reverse-mode derivative of the same recurrence, one token
at a time in reverse order (also in ``gdr_oracle.c``).

Pins: ``tests/test_oracle_pins.py`` checks ``gdr_fwd`` against closed forms,
exact rational arithmetic on tiny inputs, an independently derived chunked
(WY) evaluation, and the packing / ghost / resume invariants;
``tests/test_oracle_bwd_pins.py`` checks ``gdr_bwd`` against automatic
differentiation of an fp64 recurrence written separately in PyTorch and
against central finite differences of ``gdr_fwd``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.gdr_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, lp, i64, i64, i64, i64, i64, i64,
                                   dp, dp, dp, ctypes.c_double, ctypes.c_int]
    lib.gdr_oracle_fwd.restype = ctypes.c_int
    lib.gdr_oracle_fwd_chunks.argtypes = [dp, dp, dp, dp, dp, lp, i64, i64, i64, i64, i64, i64,
                                          dp, dp, dp, dp, ctypes.c_double, ctypes.c_int]
    lib.gdr_oracle_fwd_chunks.restype = ctypes.c_int
    lib.gdr_oracle_fwd_checkpoints.argtypes = [dp, dp, dp, dp, dp, lp, i64, i64, i64, i64, i64, i64,
                                               dp, dp, dp, dp, i64, ctypes.c_double, ctypes.c_int]
    lib.gdr_oracle_fwd_checkpoints.restype = ctypes.c_int
    lib.gdr_oracle_kda_fwd.argtypes = [dp, dp, dp, dp, dp, lp, i64, i64, i64, i64, i64, i64,
                                       dp, dp, dp, ctypes.c_double, ctypes.c_int]
    lib.gdr_oracle_kda_fwd.restype = ctypes.c_int
    lib.gdr_oracle_bwd.argtypes = [dp, dp, dp, dp, dp, lp, i64, i64, i64, i64, i64, i64,
                                   dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_double, ctypes.c_int]
    lib.gdr_oracle_bwd.restype = ctypes.c_int
    lib.gdr_oracle_threads.argtypes = [ctypes.c_int, i64]
    lib.gdr_oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = _bind(_LIB_PATH)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray], ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def threads_used(n_threads: int, n_items: int) -> int:
    """Threads ``gdr_fwd`` runs on for ``n_items`` (sequence, v-head) pairs."""
    return int(_load().gdr_oracle_threads(int(n_threads), int(n_items)))


def gdr_fwd(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None,
            ht_init=None, n_threads: int = 0, _lib_path: Optional[str] = None,
            chunk_states: bool = False, checkpoint_every: int = 64):
    """Per-token fp64 forward of the gated delta rule.

    Shapes: q, k ``[B, T, Hk, dk]``; v ``[B, T, Hv, dv]``; g, beta ``[B, T, Hv]``;
    ``cu_seqlens`` ``[N+1]`` integer offsets (requires B == 1), or None for B
    fixed-length sequences; h0 ``[N, Hv, dk, dv]`` or None for a zero state.
    ``scale`` defaults to ``dk ** -0.5``.  ``ht_init`` pre-fills the final state
    (rows of length-0 segments keep it).  Returns ``(o [B,T,Hv,dv], ht [N,Hv,dk,dv])``
    in fp64.  All inputs are taken at their exact values (bf16/fp32 upcast).
    ``_lib_path`` runs another build of the C source (the pin tests use it to
    check that deliberately broken copies of the oracle fail the pins).
    ``chunk_states=True`` also returns the state after every 64-token chunk of
    every segment, ``[NT, Hv, dk, dv]`` with chunk c of segment n at row
    ``sum(ceil(L_m / 64) for m < n) + c`` (the last chunk may be partial).
    ``checkpoint_every`` (with ``chunk_states``) replaces 64 by that many
    tokens: row ``sum(ceil(L_m / n) for m < n) + j`` holds the state after
    ``min((j + 1) * checkpoint_every, L_n)`` tokens of segment n.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or g.ndim != 3 or beta.shape != g.shape:
        raise ValueError("oracle: expected q,k [B,T,Hk,dk], v [B,T,Hv,dv], g,beta [B,T,Hv]")
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or g.shape != (B, T, Hv):
        raise ValueError("oracle: inconsistent shapes")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("oracle: cu_seqlens requires B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seq = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    h0a = None if h0 is None else _f64(h0)
    if h0a is not None and h0a.shape != (n_seq, Hv, dk, dv):
        raise ValueError("oracle: h0 must be [N, Hv, dk, dv]")
    o = np.zeros((B, T, Hv, dv), dtype=np.float64)
    if ht_init is None:
        ht = np.zeros((n_seq, Hv, dk, dv), dtype=np.float64)
    else:
        ht = _f64(ht_init).copy()
        if ht.shape != (n_seq, Hv, dk, dv):
            raise ValueError("oracle: ht_init must be [N, Hv, dk, dv]")
    lib = _load() if _lib_path is None else _bind(_lib_path)
    hck = None
    every = int(checkpoint_every)
    if every < 1:
        raise ValueError("oracle: checkpoint_every must be >= 1")
    if chunk_states:
        lens = np.maximum(np.diff(cu), 0)
        hck = np.zeros((int(((lens + every - 1) // every).sum()), Hv, dk, dv), dtype=np.float64)
    if every == 64:
        rc = lib.gdr_oracle_fwd_chunks(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(cu, ctypes.c_int64), n_seq, B * T, Hk, Hv, dk, dv,
                                       _ptr(h0a), _ptr(o), _ptr(ht), _ptr(hck), float(scale),
                                       int(n_threads))
    else:
        rc = lib.gdr_oracle_fwd_checkpoints(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                            _ptr(cu, ctypes.c_int64), n_seq, B * T, Hk, Hv, dk, dv,
                                            _ptr(h0a), _ptr(o), _ptr(ht), _ptr(hck), every,
                                            float(scale), int(n_threads))
    if rc != 0:
        raise ValueError("oracle: gdr_oracle_fwd returned %d" % rc)
    return (o, ht, hck) if chunk_states else (o, ht)


def gdr_kda_fwd(q, k, v, g, beta, cu_seqlens=None, h0=None, scale: Optional[float] = None,
                ht_init=None, n_threads: int = 0, _lib_path: Optional[str] = None):
    """Per-token fp64 forward with per-channel gates: ``g`` is ``[B, T, Hv, dk]``
    (natural-log decay of each key channel); everything else as ``gdr_fwd``.
    Returns ``(o, ht)``."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv, dk) or beta.shape != (B, T, Hv):
        raise ValueError("oracle: expected g [B, T, Hv, dk] and beta [B, T, Hv]")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("oracle: cu_seqlens requires B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seq = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    h0a = None if h0 is None else _f64(h0)
    o = np.zeros((B, T, Hv, dv), dtype=np.float64)
    ht = np.zeros((n_seq, Hv, dk, dv)) if ht_init is None else _f64(ht_init).copy()
    lib = _load() if _lib_path is None else _bind(_lib_path)
    rc = lib.gdr_oracle_kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu, ctypes.c_int64),
                                n_seq, B * T, Hk, Hv, dk, dv, _ptr(h0a), _ptr(o), _ptr(ht), float(scale),
                                int(n_threads))
    if rc != 0:
        raise ValueError("oracle: gdr_oracle_kda_fwd returned %d" % rc)
    return o, ht


def gdr_bwd(q, k, v, g, beta, do, cu_seqlens=None, h0=None, dht=None,
            scale: Optional[float] = None, dh0_init=None, n_threads: int = 0,
            _lib_path: Optional[str] = None):
    """Per-token fp64 backward of the gated delta rule forward (``gdr_fwd``).

    ``do`` ``[B, T, Hv, dv]`` and ``dht`` ``[N, Hv, dk, dv]`` (None = zero) are the
    upstream gradients of o and ht.  Returns a dict of fp64 arrays: ``dq``,
    ``dk`` ``[B, T, Hk, dk]`` (summed over the v-heads of each group), ``dv``
    ``[B, T, Hv, dv]``, ``dg``, ``dbeta`` ``[B, T, Hv]`` and ``dh0``
    ``[N, Hv, dk, dv]`` (rows of length-0 segments keep ``dh0_init``, default 0).
    """
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or \
            beta.shape != g.shape or do.shape != v.shape:
        raise ValueError("oracle: inconsistent shapes")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("oracle: cu_seqlens requires B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n_seq = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    h0a = None if h0 is None else _f64(h0)
    dhta = None if dht is None else _f64(dht)
    for name, x in (("h0", h0a), ("dht", dhta)):
        if x is not None and x.shape != (n_seq, Hv, dk, dv):
            raise ValueError("oracle: %s must be [N, Hv, dk, dv]" % name)
    out = dict(dq=np.zeros((B, T, Hk, dk)), dk=np.zeros((B, T, Hk, dk)),
               dv=np.zeros((B, T, Hv, dv)), dg=np.zeros((B, T, Hv)), dbeta=np.zeros((B, T, Hv)),
               dh0=np.zeros((n_seq, Hv, dk, dv)) if dh0_init is None else _f64(dh0_init).copy())
    lib = _load() if _lib_path is None else _bind(_lib_path)
    rc = lib.gdr_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(cu, ctypes.c_int64), n_seq, B * T, Hk, Hv, dk, dv, _ptr(h0a),
                            _ptr(do), _ptr(dhta), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), float(scale),
                            int(n_threads))
    if rc != 0:
        raise ValueError("oracle: gdr_oracle_bwd returned %d" % rc)
    return out
