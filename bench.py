"""Benchmark: learned-indexer routed sparse attention on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: key compression -> block scoring + top-k selection -> route
expansion -> sparse GQA attention forward (the S=8192 workload is forward
only).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload s8192] [--no-cpu-baseline]

``value`` is the forward attention throughput in TFLOP/s counted on
selected (query, key) pairs only: 2*(Dqk+Dv)*Hq per pair, pairs = sum of the
produced route lengths, divided by the forward kernel's time inside the
timed steps.  ``routed_queries_per_s`` is valid queries / route-pipeline
time.  Both are measured with HIP events on the stream every kernel runs on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=256)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: the hot path has no multi-GPU mode here "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import indexer_routed_block_amd as irb
    import synth

    wl = synth.WORKLOADS[args.workload]
    if wl.latent:
        raise SystemExit("the benchmark step runs the route pipeline; pick a routed workload")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.time()
    x = synth.make_inputs(wl, parts=("route", "attn"))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    d = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev, dt if k in ("kI", "qI", "q", "k", "v") else None)
         for k in ("kI", "qI", "w", "gamma", "freqs", "q", "k", "v")}
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).to(dev)
    gen_s = time.time() - t0
    S, B = wl.S, wl.B
    c, topk, window = wl.c, wl.topk, wl.window
    scale = 1.0 / math.sqrt(wl.D)

    # persistent buffers: the step allocates nothing
    L = irb.route_width(topk, c, window)
    nb = S // c
    ws_rows = S
    fused_ws = torch.empty(B * ws_rows * nb * 4, dtype=torch.uint8, device=dev)
    sel = torch.empty((B, S, topk), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, S), dtype=torch.int32, device=dev)
    dummy = torch.empty((B, 1, 1), dtype=torch.float32, device=dev)
    routes = torch.empty((B, S, L), dtype=torch.int32, device=dev)
    lens = torch.empty((B, S), dtype=torch.int32, device=dev)
    out = torch.empty((B, S, wl.Hq, wl.Dv), dtype=dt, device=dev)
    lse = torch.empty((B, wl.Hq, S), dtype=torch.float32, device=dev)
    kc = torch.empty((B, nb, wl.D_idx), dtype=torch.float32, device=dev)
    cu_blocks = None if cu is None else torch.empty(cu.numel(), dtype=torch.int32, device=dev)
    lib = irb.load_library()
    stream = torch.cuda.current_stream(dev)
    sptr = irb._stream(dev)
    lay = irb.make_layout(B, S, cu, None)
    q0 = 0 if cu is not None else min(irb.first_sparse_query(c, topk), S - 1)
    strides = irb._strides9(d["q"], d["k"], d["v"])
    P = irb._ptr

    def route_step():
        irb._check(lib.irb_compress_keys(irb.ctypes.byref(lay), c, P(d["kI"]), irb._dtype_code(d["kI"]),
                                         d["kI"].stride(0), d["kI"].stride(1), wl.D_idx, P(d["gamma"]), 1e-5,
                                         P(d["freqs"]), d["freqs"].shape[-1], P(kc), P(cu_blocks), sptr))
        if q0 > 0:
            irb._check(lib.irb_select_topk_regions(irb.ctypes.byref(lay), P(dummy), 1, 0, q0, P(cu_blocks), c, topk,
                                                   P(sel), P(cnt), sptr))
        irb._check(lib.irb_route_topk_fused(irb.ctypes.byref(lay), P(d["qI"]), irb._dtype_code(d["qI"]), wl.H_idx,
                                            wl.D_idx, P(d["w"]), P(kc), P(cu_blocks), c, 1.0 / math.sqrt(wl.D_idx),
                                            topk, q0, S, P(sel), P(cnt), P(fused_ws), fused_ws.numel(), sptr))
        irb._check(lib.irb_expand_and_compact_routes(irb.ctypes.byref(lay), P(sel), P(cnt), topk, c, window,
                                                     P(cu_blocks), L, P(routes), P(lens), sptr))

    def attn_step():
        irb._check(lib.irb_sparse_gqa_attention_fwd(P(d["q"]), P(d["k"]), P(d["v"]), irb._dtype_code(d["q"]), strides,
                                                    P(routes), P(lens), B, S, S, L, wl.Hq, wl.Hkv, wl.D, wl.Dv, scale,
                                                    P(out), P(lse), sptr))

    for _ in range(args.warmup):
        route_step()
        attn_step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        route_step()
        ev[i][1].record(stream)
        attn_step()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    route_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    attn_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    step_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in range(args.steps)]

    lens_h = lens.cpu().numpy().astype(np.int64)
    pairs = int(lens_h.sum())
    valid_q = int((lens_h > 0).sum())
    fwd_flop = 2.0 * (wl.D + wl.Dv) * wl.Hq * pairs
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    route_avg_s = float(np.mean(route_ms)) / 1e3
    tflops = fwd_flop / attn_avg_s / 1e12
    qps = valid_q / route_avg_s

    result = {
        "metric": "sparse-attn fwd TFLOP/s (selected pairs) + routed queries/s, S=8192",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "routed_queries_per_s": round(qps, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 4),
        "ms_route": round(float(np.mean(route_ms)), 4),
        "ms_attn_fwd": round(float(np.mean(attn_ms)), 4),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": B, "S": S, "H_idx": wl.H_idx, "D_idx": wl.D_idx, "c": c, "topk": topk,
            "window": window, "route_width": L, "Hq": wl.Hq, "Hkv": wl.Hkv, "Dqk": wl.D, "Dv": wl.Dv,
            "selected_pairs": pairs, "valid_queries": valid_q,
        },
        "roofline": {
            "kernel": "attn_fwd_kernel (gather, G<=16)",
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 5),
            "traffic": None,
            "algorithmic_flop_per_launch": fwd_flop,
            "avg_launch_ms": round(attn_avg_s * 1e3, 5),
            "gathered_GBps": round(2.0 * (wl.D + wl.Dv) * wl.Hkv * pairs / attn_avg_s / 1e9, 1),
        },
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_sample_rows)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, x, n_rows):
    """The FP64 oracle on a bounded sample: n_rows query rows spread over the sequence.

    Route pipeline (compress all blocks, then score / select / expand the
    sampled rows) and the attention forward of the same rows, each timed
    with perf_counter on this host's cores.
    """
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    S = wl.S
    rows = np.linspace(S // 4, S - 1, n_rows).astype(int)
    t0 = time.perf_counter()
    kc, _ = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c)
    sel = np.full((1, S, wl.topk), -1, dtype=np.int32)
    cnt = np.zeros((1, S), dtype=np.int32)
    for t in rows:
        s = oracle.indexer_scores(x["qI"], x["w"], kc, wl.c, q0=int(t), q1=int(t) + 1)
        st, ct = oracle.select_topk(s, wl.c, wl.topk, q0=int(t), S=S)
        sel[0, t], cnt[0, t] = st[0, 0], ct[0, 0]
    routes, _ = oracle.expand_routes(sel, cnt, wl.c, wl.window, wl.topk, rows=[(0, int(t)) for t in rows])
    route_s = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.attention_fwd(x["q"], x["k"], x["v"], routes, rows=[(0, int(t)) for t in rows])
    attn_s = time.perf_counter() - t1
    pairs = int((routes[0, rows] >= 0).sum())
    flop = 2.0 * (wl.D + wl.Dv) * wl.Hq * pairs
    return {"value": round(flop / attn_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} query rows (evenly spaced from S/4 to S-1) of the {wl.name} workload; FP64 NumPy; "
                      f"attention fwd {attn_s:.2f} s, route pipeline {route_s:.2f} s "
                      f"({n_rows / route_s:.1f} routed queries/s incl. full key compression)"}


if __name__ == "__main__":
    main()
