"""Seeded synthetic inputs for the gated delta rule forward pass.

This module holds no arithmetic of the method itself: it only draws inputs.
Both the oracle-side tests and the HIP path take their inputs from here.

Distributions (the pages' own test setup, "FlashQLA GDN backend produces
different tokens from FLA Triton", maintainer reply: q and k L2-normalised,
v Gaussian), completed by the workload definitions below:

* q, k ~ N(0, 1), then L2-normalised over the head dimension, per token and head;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)),  g = logsigmoid(N(0, 1))  (one value per token and v-head);
* h0 ~ 0.1 * N(0, 1) per sequence and v-head (standard deviation 0.1), fp32.

Values are drawn with ``numpy.random.Generator(PCG64(seed))`` in the order
lengths -> q -> k -> v -> g -> beta -> h0, computed in fp32/fp64 and then rounded
once to the storage dtype (bf16 with round-to-nearest-even, or fp32).  The
arrays returned are float32 arrays whose values are exactly representable in
the storage dtype, so the oracle and the GPU see the same bits.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int                   # fixed-length rows (packed workloads: 1)
    seq_len: int                 # tokens per row (packed: total tokens)
    hk: int                      # q/k heads
    hv: int                      # v heads
    dk: int
    dv: int
    dtype: str                   # storage dtype of q, k, v, g, beta, o: "bf16" | "fp32"
    seg_range: Optional[tuple] = None   # (lo, hi) inclusive segment lengths (packed)
    n_segments: Optional[int] = None    # fixed count of drawn segments (else fill seq_len)
    ghosts: int = 0              # trailing length-0 segments appended to cu_seqlens
    with_h0: bool = True
    seed: int = 0
    description: str = ""


# The five workloads: the parity cases and the benchmark workload.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_fp32_T128_H2_d64", 1, 128, 2, 2, 64, 64, "fp32", with_h0=False, seed=1001,
             description="B=1, T=128 (2 chunks of 64), H=2, dk=dv=64, fp32, zero initial state"),
    Workload("fixed_B4_T512_H16_d128", 4, 512, 16, 16, 128, 128, "bf16", seed=1002,
             description="B=4, T=512, H=16, dk=dv=128, bf16, h0 ~ 0.1 N(0,1)"),
    Workload("varlen8_ghost8_H32_d128", 1, 0, 32, 32, 128, 128, "bf16", seg_range=(1, 512),
             n_segments=8, ghosts=8, seed=1003,
             description="8 segments of lengths U{1..512} + 8 trailing length-0 segments, "
                         "H=32, dk=dv=128, bf16, h0 per segment"),
    Workload("long_T20468_H16_d128", 1, 20468, 16, 16, 128, 128, "bf16", with_h0=False, seed=1004,
             description="B=1, T=20468 (last chunk 52 tokens), H=16, dk=dv=128, bf16, zero state"),
    Workload("packed64k_gqa_Hk16_Hv32_d128", 1, 65536, 16, 32, 128, 128, "bf16",
             seg_range=(256, 8192), seed=1005,
             description="T=65536 packed into segments of lengths U{256..8192} (last one takes "
                         "the remainder), Hk=16 shared by Hv=32 (GQA 2:1), dk=dv=128, bf16, "
                         "h0 per segment"),
]}

WORKLOAD_ORDER: List[str] = list(WORKLOADS)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x)
    raise ValueError("unknown dtype %r" % dtype)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...d,...d->...", x, x, dtype=np.float64))
    return (x / n[..., None]).astype(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-x)), np.exp(x) / (1.0 + np.exp(x)))


def draw_lengths(rng: np.random.Generator, w: Workload) -> Optional[List[int]]:
    """Segment lengths of a packed workload (None for fixed-length rows)."""
    if w.seg_range is None:
        return None
    lo, hi = w.seg_range
    if w.n_segments is not None:
        return [int(x) for x in rng.integers(lo, hi, size=w.n_segments, endpoint=True)]
    out, total = [], 0
    while total < w.seq_len:
        L = int(rng.integers(lo, hi, endpoint=True))
        L = min(L, w.seq_len - total)      # the last segment takes the remainder
        out.append(L)
        total += L
    return out


def generate(w: Workload, seed: Optional[int] = None, lengths: Optional[List[int]] = None,
             g_mode: str = "logsigmoid", beta_mode: str = "sigmoid") -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with float32 arrays ``q, k [B,T,Hk,dk]``, ``v [B,T,Hv,dv]``,
    ``g, beta [B,T,Hv]``, ``h0 [N,Hv,dk,dv]`` (or None), int32 ``cu_seqlens``
    (or None for fixed-length rows), the list of real segment ``lengths``,
    and ``scale = dk ** -0.5``.

    ``g_mode``: "logsigmoid" (default), "zero" (no decay) or "logsigmoid/16"
    (slow decay) — the latter two are stress variants of the same shapes.
    ``beta_mode``: "sigmoid" (default) or "zero".
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    drawn = draw_lengths(rng, w)
    if lengths is not None:
        drawn = list(lengths)
    if drawn is None:
        B, T = w.batch, w.seq_len
        n_seq = B
        cu = None
    else:
        B, T = 1, int(sum(drawn))
        offs = np.concatenate([[0], np.cumsum(drawn, dtype=np.int64)])
        offs = np.concatenate([offs, np.full(w.ghosts, offs[-1], dtype=np.int64)])
        cu = offs.astype(np.int32)
        n_seq = len(drawn) + w.ghosts
    dt = w.dtype
    q = _store(_l2norm(rng.standard_normal((B, T, w.hk, w.dk), dtype=np.float32)), dt)
    k = _store(_l2norm(rng.standard_normal((B, T, w.hk, w.dk), dtype=np.float32)), dt)
    v = _store(rng.standard_normal((B, T, w.hv, w.dv), dtype=np.float32), dt)
    g_raw = rng.standard_normal((B, T, w.hv), dtype=np.float32)
    b_raw = rng.standard_normal((B, T, w.hv), dtype=np.float32)
    if g_mode == "logsigmoid":
        g = _logsigmoid(g_raw)
    elif g_mode == "logsigmoid/16":
        g = _logsigmoid(g_raw) / 16.0
    elif g_mode == "zero":
        g = np.zeros_like(g_raw, dtype=np.float64)
    else:
        raise ValueError(g_mode)
    beta = _sigmoid(b_raw) if beta_mode == "sigmoid" else np.zeros_like(b_raw, dtype=np.float64)
    g = _store(g, dt)
    beta = _store(beta, dt)
    h0 = None
    if w.with_h0:
        h0 = (0.1 * rng.standard_normal((n_seq, w.hv, w.dk, w.dv), dtype=np.float32)).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu_seqlens=cu,
                lengths=drawn if drawn is not None else [T] * B,
                scale=float(w.dk) ** -0.5, dtype=dt, workload=w.name)


def random_lengths_case(seed: int, n_real: int, lo: int, hi: int, ghost_slots: int,
                        hk: int, hv: int, d: int, dtype: str = "bf16", with_h0: bool = True) -> dict:
    """A packed case with ghosts placed at random slots among real segments."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [int(x) for x in rng.integers(lo, hi, size=n_real, endpoint=True)]
    slots = sorted(int(s) for s in rng.integers(0, n_real + 1, size=ghost_slots))
    seq = []
    for i, L in enumerate(lens):
        seq.extend([0] * sum(1 for s in slots if s == i))
        seq.append(L)
    seq.extend([0] * sum(1 for s in slots if s == n_real))
    w = Workload("random", 1, 0, hk, hv, d, d, dtype, seg_range=(lo, hi), n_segments=len(seq),
                 with_h0=with_h0, seed=seed + 1)
    return generate(w, lengths=seq)


def generate_grads(case: dict, seed: int) -> dict:
    """Upstream gradients for a backward pass over ``case`` (a dict from
    ``generate``): ``do`` ~ N(0, 1) of o's shape, rounded to the case's dtype,
    and ``dht`` ~ N(0, 1) of the final state's shape, fp32.  Drawn with
    ``PCG64(seed)`` in the order do -> dht."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = case["v"]
    n_seq = (len(case["cu_seqlens"]) - 1) if case["cu_seqlens"] is not None else v.shape[0]
    do = _store(rng.standard_normal(v.shape, dtype=np.float32), case["dtype"])
    dht = rng.standard_normal((n_seq, v.shape[2], case["q"].shape[3], v.shape[3]),
                              dtype=np.float32).astype(np.float32)
    return dict(do=do, dht=dht)


def generate_kda_gates(case: dict, seed: int, scale: float = 1.0) -> "np.ndarray":
    """Per-channel log-gates for the per-channel-gate variant of ``case``:
    ``scale * logsigmoid(N(0, 1))`` of shape ``[B, T, Hv, dk]`` (drawn with
    ``PCG64(seed)``), rounded to the case's dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v, q = case["v"], case["q"]
    x = rng.standard_normal(v.shape[:3] + (q.shape[3],), dtype=np.float32)
    return _store(scale * _logsigmoid(x), case["dtype"])
