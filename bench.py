"""Benchmark of the chunked gated delta rule forward on one MI355X.

A step is one full forward (chunk preparation + the fused chunk kernel) over
the packed 64k-token workload: T = 65536 tokens in segments of seeded lengths
U{256..8192}, 16 q/k heads shared by 32 v-heads, head dim 128, bf16 inputs,
fp32 state, per-segment initial state.  Inputs are resident in HBM before the
timed region.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk-fwd tokens/sec on 1 MI355X (H=32,d=128); % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
CHUNK = 64


def flops_chunk(dk: int, dv: int) -> int:
    """Chunk-form flops per (token, v-head): K K^T, W, U, W H, K^T Vnew, Q H,
    Q K^T and P Vnew with every 64-wide intra-chunk block counted in full."""
    return 6 * dk * dv + 2 * CHUNK * (3 * dk + 2 * dv)


def flops_min(dk: int, dv: int, r: int) -> float:
    """The same with triangles exploited exactly, the 64x64 inverse included and
    K K^T / Q K^T shared by the r v-heads of a q/k head."""
    C = CHUNK
    kk = (C - 1) / 2 * 2 * dk / r           # strict lower K K^T, per token
    qk = (C + 1) / 2 * 2 * dk / r           # inclusive lower Q K^T
    tri_apply = (C + 1) / 2 * 2 * (dk + dv)  # unit-lower T applied to [K|V]
    inv = (C - 1) * (C - 2) / 3             # per token share of the inverse
    state = 4 * dk * dv + 2 * dk * dv        # W H, K^T Vnew, Q H
    pv = (C + 1) / 2 * 2 * dv               # inclusive lower P Vnew
    return kk + qk + tri_apply + inv + state + pv


def bytes_alg(T: int, N: int, hk: int, hv: int, dk: int, dv: int, in_bytes: int, gate_bytes: int) -> int:
    """Every input read once and every output written once."""
    per_tok = hk * 2 * dk * in_bytes + hv * (2 * dv * in_bytes + 2 * gate_bytes)
    return T * per_tok + N * hv * 2 * dk * dv * 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="packed64k_gqa_Hk16_Hv32_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="v-heads of every segment the CPU baseline runs (a bounded sample)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_fwd_packed64k.json"))
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import chunked_gated_delta_fwd_amd as gdr
    import gdr_inputs as gi

    if not os.path.exists(gdr.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    gdr.library()
    w = gi.WORKLOADS[args.workload]
    d = gi.generate(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def put(x, dtype):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dtype)

    q, k, v = put(d["q"], dt), put(d["k"], dt), put(d["v"], dt)
    g, beta = put(d["g"], dt), put(d["beta"], dt)
    cu = put(d["cu_seqlens"], torch.int32)
    h0 = put(d["h0"], torch.float32)
    B, T = q.shape[0], q.shape[1]
    N = (cu.shape[0] - 1) if cu is not None else B
    o = torch.empty((B, T, w.hv, w.dv), dtype=dt, device=dev)
    ht = torch.empty((N, w.hv, w.dk, w.dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        gdr.chunk_fwd(q, k, v, g, beta, cu, h0, scale=d["scale"], o=o, ht=ht)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = sum(per_call_ms) / len(per_call_ms)

    tokens = B * T
    in_bytes = 2 if w.dtype == "bf16" else 4
    f_chunk = flops_chunk(w.dk, w.dv) * tokens * w.hv
    f_min = flops_min(w.dk, w.dv, w.hv // w.hk) * tokens * w.hv
    nbytes = bytes_alg(tokens, N, w.hk, w.hv, w.dk, w.dv, in_bytes, in_bytes)
    achieved_tflops = f_chunk / (launch_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            if tj.get("workload") == w.name and tj.get("kernel_source_sha") == kernel_source_sha():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": tokens, "segments": N, "hk": w.hk, "hv": w.hv,
                   "dk": w.dk, "dv": w.dv, "chunk": CHUNK, "seed": w.seed},
        "roofline": {
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel": "gdr_fwd_kernel<128,bf16,bf16> (+ gdr_prepare_kernel in the same call)",
            "flops_per_launch": f_chunk,
            "launch_ms": launch_ms,
        },
        "mfma_frac_fmin": f_min / (launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "hbm": {"bytes_alg": nbytes, "achieved_GBps": nbytes / (launch_ms * 1e-3) / 1e9,
                "frac": nbytes / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_heads)
    print(json.dumps(out), flush=True)


def kernel_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ("gdr_kernels.hip", "gdr_api.cpp", "gdr_internal.h"):
        with open(os.path.join(ROOT, "chunked_gated_delta_fwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(d, w, heads: int) -> dict:
    """The fp64 oracle on the host cores over a bounded sample of the same
    workload: every segment, the first `heads` v-heads (with their q/k heads)."""
    import numpy as np

    import oracle
    heads = max(1, min(heads, w.hv))
    r = w.hv // w.hk
    hk_n = (heads + r - 1) // r
    sub = dict(q=d["q"][:, :, :hk_n], k=d["k"][:, :, :hk_n], v=d["v"][:, :, :heads],
               g=d["g"][:, :, :heads], beta=d["beta"][:, :, :heads])
    h0 = None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, :heads])
    cu = d["cu_seqlens"]
    n_items = (len(cu) - 1 if cu is not None else d["q"].shape[0]) * heads
    threads = oracle.threads_used(0, n_items)
    t0 = time.perf_counter()
    oracle.gdr_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], cu, h0, scale=d["scale"])
    sec = time.perf_counter() - t0
    tokens = d["q"].shape[0] * d["q"].shape[1]
    # tokens/s of the whole workload (all Hv heads) at the sampled rate
    return {"value": tokens * heads / w.hv / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "all %d tokens, v-heads 0..%d of %d (%.1f%% of the work), %.2f s wall"
                      % (tokens, heads - 1, w.hv, 100.0 * heads / w.hv, sec)}


if __name__ == "__main__":
    main()
