"""Benchmark of the chunked gated delta rule forward on one MI355X.

A step is one full forward (chunk preparation + the fused chunk kernel) over
the packed 64k-token workload: T = 65536 tokens in segments of seeded lengths
U{256..8192}, 16 q/k heads shared by 32 v-heads, head dim 128, bf16 inputs,
fp32 state, per-segment initial state.  Inputs are resident in HBM before the
timed region.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--settle-calls S] [--workload NAME] [--no-cpu-baseline]

Before the warm-up steps, --settle-calls (default 200) untimed steps run back
to back: after idle the GPU's clock first drops and needs about 100 calls of
sustained work to settle (see profiles/fwd_packed64k_clock_transient.md), and
the timed steps are meant to show the steady state.  The count is reported in
the JSON line as settle_calls.

Two helper modes feed the HBM traffic figure of the roofline object:
  python bench.py --copy-probe-mib M     a plain device copy of M MiB (one
                                         elementwise kernel that reads M MiB
                                         and writes M MiB), run under
                                         rocprofv3 --pmc to calibrate the
                                         FETCH_SIZE / WRITE_SIZE counters;
  python bench.py --traffic-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --copy-probe-mib M
                                         reads the counter CSVs of those four
                                         rocprofv3 runs and writes the traffic
                                         summary that later bench runs report.
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


def flops_bwd(dk: int, dv: int) -> int:
    """Backward flops per (token, v-head), every 64-wide block counted in full:
    the per-chunk preparation (K K^T, Q K^T, w = T K, dU0 = P^T dO), the reverse
    chain (K dS', Q^T dO, w^T dU) and the per-chunk gradients (K S, U = T W,
    T^T dU, dO S^T, dW S^T, U dS'^T, dO U^T, dW U^T and four 64-deep products
    with K or Q), plus the forward recompute (flops_chunk)."""
    state = 8 * 2 * dk * dv                  # eight products over a full state, per token
    intra = 2 * CHUNK * (7 * dk + 5 * dv)    # twelve 64 x 64 x d products, per token
    return state + intra + flops_chunk(dk, dv)


def flops_kda(dk: int, dv: int) -> int:
    """Per-channel-gate forward flops per (token, v-head), every 64-wide block
    counted in full: A and P (two 64 x 64 x dk), k~ S and q~ S, U = T W and P U,
    and k^^T U (three full-state products)."""
    return 6 * dk * dv + 2 * CHUNK * (2 * dk + 2 * dv)


def bytes_alg(T: int, N: int, hk: int, hv: int, dk: int, dv: int, in_bytes: int, gate_bytes: int) -> int:
    """Every input read once and every output written once."""
    per_tok = hk * 2 * dk * in_bytes + hv * (2 * dv * in_bytes + 2 * gate_bytes)
    return T * per_tok + N * hv * 2 * dk * dv * 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="packed64k_gqa_Hk16_Hv32_d128")
    ap.add_argument("--settle-calls", type=int, default=200,
                    help="back-to-back steps run before the warm-up steps, untimed, so that the GPU's "
                         "clock has left the transient that follows a burst of work after idle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="v-heads of every segment the CPU baseline runs (a bounded sample)")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "fwd_packed64k_traffic.txt"))
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR", default=None)
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="time gdr_decode_step for B sequences with the workload's heads "
                         "(one token each, state in place), against the HBM roofline")
    ap.add_argument("--kda", action="store_true",
                    help="time gdr_chunk_kda_fwd (one log-gate per key channel, seeded like g) "
                         "for the workload, against the MFMA roofline of its flops")
    ap.add_argument("--backward", action="store_true",
                    help="time gdr_chunk_bwd (forward recompute and all gradients) for the workload, "
                         "against the MFMA roofline of the backward flops")
    ap.add_argument("--checkpoints", action="store_true",
                    help="time gdr_chunk_fwd_checkpoints (state after every chunk written); "
                         "reported against the HBM roofline")
    return ap.parse_args()


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    w = gi.WORKLOADS[args.workload]
    if args.decode:
        bench_decode(args, w)
        return
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

    nt_chunks = sum((L + CHUNK - 1) // CHUNK for L in d["lengths"])
    if args.kda:
        gk = put(gi.generate_kda_gates(d, seed=w.seed + 3), dt)

        def step():
            gdr.chunk_kda_fwd(q, k, v, gk, beta, cu, h0, scale=d["scale"], o=o, ht=ht)
    elif args.backward:
        import gdr_inputs
        gr = gdr_inputs.generate_grads(d, seed=w.seed + 7)
        do, dht = put(gr["do"], dt), put(gr["dht"], torch.float32)
        bufs = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                    dg=torch.empty((B, T, w.hv), dtype=torch.float32, device=dev),
                    dbeta=torch.empty((B, T, w.hv), dtype=torch.float32, device=dev),
                    dh0=torch.empty((N, w.hv, w.dk, w.dv), dtype=torch.float32, device=dev))

        def step():
            gdr.chunk_bwd(q, k, v, g, beta, do, cu, h0, dht, scale=d["scale"], **bufs)
    elif args.checkpoints:
        rows = ((T + CHUNK - 1) // CHUNK + N) if cu is not None else B * ((T + CHUNK - 1) // CHUNK)
        hck = torch.empty((rows, w.hv, w.dk, w.dv), dtype=torch.float32, device=dev)

        def step():
            gdr.chunk_fwd_checkpoints(q, k, v, g, beta, cu, h0, scale=d["scale"], o=o, ht=ht, h_chunks=hck)
    else:
        def step():
            gdr.chunk_fwd(q, k, v, g, beta, cu, h0, scale=d["scale"], o=o, ht=ht)

    # Events are created before the warm-up: creating them after it would
    # leave the GPU idle long enough to restart its clock transient.  That
    # transient: after idle the first two or three calls run at full clock,
    # then the clock drops by up to a third and takes about 100 calls to settle
    # (per-call times and kernel durations in profiles/); so the warm-up steps
    # are preceded by settle_calls back-to-back steps, and the timed steps
    # measure the steady state a continuously running caller sees.
    #
    # Two events bracket the K timed steps on the launch stream (timing
    # events between consecutive calls left the GPU idle between them, which
    # a caller running the steps back to back does not pay).  launch_ms is
    # the average time per call on the stream: both kernels of the call and
    # the dispatch gap between calls included.
    stream = torch.cuda.current_stream(dev)
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    # torch creates an event's HIP object at its first record: record both
    # once now, so that no event is created inside the timed region
    ev_start.record(stream)
    ev_end.record(stream)
    for _ in range(args.settle_calls):
        step()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for _ in range(args.steps):
        step()
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = ev_start.elapsed_time(ev_end) / args.steps

    tokens = B * T
    in_bytes = 2 if w.dtype == "bf16" else 4
    f_chunk = flops_chunk(w.dk, w.dv) * tokens * w.hv
    f_min = flops_min(w.dk, w.dv, w.hv // w.hk) * tokens * w.hv
    nbytes = bytes_alg(tokens, N, w.hk, w.hv, w.dk, w.dv, in_bytes, in_bytes)
    achieved_tflops = f_chunk / (launch_ms * 1e-3) / 1e12
    traffic = read_traffic(args.traffic_file, w.name)

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
        "settle_calls": args.settle_calls,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel": "gdr_fwd_kernel<128,bf16,bf16> (+ gdr_order_kernel in the same call)",
            "flops_per_launch": f_chunk,
            "launch_ms": launch_ms,
        },
        "mfma_frac_fmin": f_min / (launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "hbm": {"bytes_alg": nbytes, "achieved_GBps": nbytes / (launch_ms * 1e-3) / 1e9,
                "frac": nbytes / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "cpu_baseline": None,
    }
    if args.kda:
        fk = flops_kda(w.dk, w.dv) * tokens * w.hv
        gbytes = tokens * w.hv * w.dk * in_bytes
        out["config"]["kda"] = True
        out["roofline"] = {"bound": "mfma", "achieved": fk / (launch_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": fk / (launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "traffic": None, "kernel": "gdr_kda_fwd_kernel<128,bf16,bf16> (+ gdr_prepare_kernel)",
                           "flops_per_launch": fk, "launch_ms": launch_ms}
        out.pop("mfma_frac_fmin")
        out["hbm"] = {"bytes_alg": nbytes + gbytes, "achieved_GBps": (nbytes + gbytes) / (launch_ms * 1e-3) / 1e9,
                      "frac": (nbytes + gbytes) / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    if args.backward:
        fb = flops_bwd(w.dk, w.dv) * tokens * w.hv
        out["config"]["backward"] = True
        out["roofline"] = {"bound": "mfma", "achieved": fb / (launch_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": fb / (launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "traffic": None,
                           "kernel": "gdr_chunk_bwd: gdr_prepare_kernel, gdr_fwd_kernel<checkpoints>, "
                                     "gdr_bwd_prep_kernel, gdr_bwd_chain_kernel, gdr_bwd_grads_kernel",
                           "flops_per_launch": fb, "launch_ms": launch_ms}
        out.pop("mfma_frac_fmin")
        out.pop("hbm")
    if args.checkpoints:
        # the same call plus 4*dk*dv bytes written per (chunk, v-head): HBM bound
        ck_bytes = nt_chunks * w.hv * w.dk * w.dv * 4
        tot = nbytes + ck_bytes
        out["config"]["checkpoints"] = True
        out["roofline"] = {"bound": "hbm", "achieved": tot / (launch_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": tot / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "traffic": None,
                           "kernel": "gdr_fwd_kernel<128,bf16,bf16,checkpoints> (+ gdr_prepare_kernel)",
                           "bytes_per_launch": tot, "checkpoint_bytes": ck_bytes, "launch_ms": launch_ms}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_heads)
    print(json.dumps(out), flush=True)


def bench_decode(args, w):
    """Decode-step throughput: B sequences x Hv heads, one token each, the
    fp32 state read and written in place (HBM bound)."""
    import torch
    import chunked_gated_delta_fwd_amd as gdr
    B, d = args.decode, w.dk
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    rnd = lambda *shape: torch.randn(*shape, generator=gen)
    q = torch.nn.functional.normalize(rnd(B, w.hk, d), dim=-1).to(dev, dt)
    k = torch.nn.functional.normalize(rnd(B, w.hk, d), dim=-1).to(dev, dt)
    v = rnd(B, w.hv, d).to(dev, dt)
    g = torch.nn.functional.logsigmoid(rnd(B, w.hv)).to(dev, dt)
    beta = torch.sigmoid(rnd(B, w.hv)).to(dev, dt)
    h = (0.1 * rnd(B, w.hv, d, d)).to(dev)
    o = torch.empty((B, w.hv, d), dtype=dt, device=dev)
    # one decode kernel takes tens of microseconds, less than the host needs
    # to marshal a call, so the steps are captured in a graph (20 per replay)
    # and replayed; the step has no allocation and no memset to capture
    per = 20
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(3):
            gdr.decode_step(q, k, v, g, beta, h, o=o)
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per):
            gdr.decode_step(q, k, v, g, beta, h, o=o)
    reps = max(1, args.steps // per)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for _ in range(max(1, args.warmup // per)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        graph.replay()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = sum(s.elapsed_time(e) for s, e in ev) / len(ev) / per
    args.steps = reps * per
    eb = 2 if w.dtype == "bf16" else 4
    nbytes = B * w.hv * (2 * d * d * 4 + 2 * d * eb + 2 * eb) + B * w.hk * 2 * d * eb
    out = {"metric": "GDN decode-step tokens/sec on 1 MI355X (one token per sequence)",
           "value": B / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "timing": "graph of %d steps per replay" % per,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
           "data": "synthetic",
           "config": {"workload": "decode_B%d_Hk%d_Hv%d_d%d" % (B, w.hk, w.hv, d), "batch": B, "hk": w.hk,
                      "hv": w.hv, "d": d},
           "roofline": {"bound": "hbm", "achieved": nbytes / (launch_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": nbytes / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "traffic": None,
                        "kernel": "gdr_decode_kernel", "bytes_per_launch": nbytes, "launch_ms": launch_ms},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


FWD_KERNEL = "gdr_fwd_kernel"
COPY_KERNEL = "neg_kernel"


def copy_probe(mib: int):
    """A plain copy of known size: torch's elementwise negation of an fp32
    buffer into another reads and writes mib MiB once each."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4}), flush=True)


def _counter_rows(d: str, counter: str, kernel_substr: str):
    """Per-dispatch values of one counter for the kernels whose name contains
    kernel_substr, from a rocprofv3 --pmc run written with -f csv under d."""
    import csv
    import glob
    vals = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % d)
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter or kernel_substr not in row.get("Kernel_Name", ""):
                    continue
                key = (fn, row.get("Dispatch_Id"))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit("no %s rows for kernels matching %r under %s" % (counter, kernel_substr, d))
    return list(vals.values())


def traffic_summary(args):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused kernel,
    each divided by the factor the same counter reads on the copy probe
    (counter bytes / true bytes), written as key: value lines."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.traffic_summary
    if not args.copy_probe_mib:
        raise SystemExit("--traffic-summary needs --copy-probe-mib (the size the copy probe ran with)")
    true_bytes = args.copy_probe_mib * (1 << 20)
    avg = lambda xs: sum(xs) / len(xs)
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE", FWD_KERNEL)
    write = _counter_rows(write_dir, "WRITE_SIZE", FWD_KERNEL)
    cfetch = _counter_rows(cfetch_dir, "FETCH_SIZE", COPY_KERNEL)
    cwrite = _counter_rows(cwrite_dir, "WRITE_SIZE", COPY_KERNEL)
    f_fetch = avg(cfetch) * 1024.0 / true_bytes
    f_write = avg(cwrite) * 1024.0 / true_bytes
    fetch_b = avg(fetch) * 1024.0 / f_fetch
    write_b = avg(write) * 1024.0 / f_write
    import gdr_inputs as gi
    w = gi.WORKLOADS[args.workload]
    lines = [
        "# HBM traffic of %s on %s (rocprofv3 --pmc, KiB per dispatch)" % (FWD_KERNEL, w.name),
        "# made by four counter runs, one counter each, then this summary:",
        "#   rocprofv3 --pmc FETCH_SIZE -f csv -d FETCH_DIR -o fwd -- "
        "python3 bench.py --steps 3 --warmup 1 --settle-calls 0 --no-cpu-baseline",
        "#   rocprofv3 --pmc WRITE_SIZE -f csv -d WRITE_DIR -o fwd -- "
        "python3 bench.py --steps 3 --warmup 1 --settle-calls 0 --no-cpu-baseline",
        "#   rocprofv3 --pmc FETCH_SIZE -f csv -d COPY_FETCH_DIR -o copy -- "
        "python3 bench.py --copy-probe-mib %d" % args.copy_probe_mib,
        "#   rocprofv3 --pmc WRITE_SIZE -f csv -d COPY_WRITE_DIR -o copy -- "
        "python3 bench.py --copy-probe-mib %d" % args.copy_probe_mib,
        "#   python3 bench.py --traffic-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR "
        "--copy-probe-mib %d" % args.copy_probe_mib,
        "workload: %s" % w.name,
        "kernel_source_sha: %s" % kernel_source_sha(),
        "fwd_dispatches: %d" % len(fetch),
        "fwd_fetch_kib_avg: %.1f" % avg(fetch),
        "fwd_write_kib_avg: %.1f" % avg(write),
        "copy_probe_bytes: %d" % true_bytes,
        "copy_dispatches: %d" % len(cfetch),
        "copy_fetch_kib_avg: %.1f" % avg(cfetch),
        "copy_write_kib_avg: %.1f" % avg(cwrite),
        "fetch_factor: %.4f" % f_fetch,
        "write_factor: %.4f" % f_write,
        "fwd_fetch_bytes: %.0f" % fetch_b,
        "fwd_write_bytes: %.0f" % write_b,
        "bytes_per_launch: %.0f" % (fetch_b + write_b),
    ]
    with open(args.traffic_file, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(path: str, workload: str):
    """bytes_per_launch of the traffic summary, or None when it is missing or
    was taken on another workload or another version of the kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("workload") != workload or kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ("gdr_kernels.hip", "gdr_device.h", "gdr_api.cpp", "gdr_internal.h"):
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
