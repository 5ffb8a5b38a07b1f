"""Benchmark: learned-indexer routed sparse attention on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM, every stage a call of the C ABI on one stream:

* routed workloads: key compression -> block scoring + top-k selection
  (fused, bounded score chunks; with shared routes the raw index queries'
  RMSNorm + RoPE runs inside the score kernel's query loads) -> route
  expansion -> sparse GQA attention
  forward, and, where the workload trains (packed 32768, 131072), reverse
  block lists -> attention backward;
* latent workload: index compaction -> attention forward -> reverse lists
  -> backward.

Calls whose outputs the step does not read (index-query preparation, the
selection's region bitmap, the full/partial split of the reverse lists) are
timed after the step, outside it, under ``aux_calls_outside_step``.

Prints one JSON line.  ``value`` is the forward attention throughput in
TFLOP/s counted on selected (query, key) pairs only: 2*(Dqk+Dv)*Hq per pair,
pairs = sum of the produced route lengths, divided by the forward call's
time.  ``routed_queries_per_s`` is valid queries / route-pipeline time.
``stages`` gives every call's mean time and its roofline fraction.  All
times come from HIP events recorded on the stream the kernels run on.

    python bench.py [--steps K] [--warmup W] [--workload s8192|varlen|long|latent|tiny]
                    [--no-cpu-baseline] [--copy-probe-mib N] [--route-groups R]

``--route-groups R`` (R = the workload's KV head count) runs the same step
with one selection and one route per KV group: the workload's index heads
split into R groups of H_idx / R, grouped fused scoring / selection, routes
[R, B, S, L] read per KV head by the attention calls.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
FP32_VALU_PEAK_TFLOPS = 157.3      # MI355X fp32 vector (published)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_s8192_hbm_traffic.json")
# the forward call's kernels: route-bit packing and the attention kernels
FWD_SOURCES = [os.path.join(ROOT, "indexer_routed_block_amd", "csrc", f)
               for f in ("attn_fwd.hip", "bitmap.hip", "irb_internal.hpp", "irb_common.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=3072)
    ap.add_argument("--route-groups", type=int, default=1,
                    help="1: one route per query for all heads; Hkv: one selection and route per KV group")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: HBM rate of the token-streaming kernels (key compression, "
                         "index-query preparation) over sequence lengths 8K..2M")
    ap.add_argument("--peaks", action="store_true",
                    help="instead of the step: achievable bf16 GEMM rate (vendor library) and device copy bandwidth")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (HBM counter calibration)")
    ap.add_argument("--cold", action="store_true",
                    help="cold-cache timing: write a 512 MiB buffer before every timed call, so that L2 and the "
                         "256 MiB Infinity Cache hold none of its inputs; ms_per_step is then the sum of the stages")
    return ap.parse_args()


def _layout_counts(wl, S, cu):
    """Host metadata: per-token visible complete blocks nb(t) and validity (doc-local positions)."""
    import numpy as np
    pos = np.zeros(S, dtype=np.int64)
    valid = np.zeros(S, dtype=bool)
    if cu is None:
        pos[:] = np.arange(S)
        valid[:] = True
    else:
        for d in range(len(cu) - 1):
            a, e = int(cu[d]), int(cu[d + 1])
            pos[a:e] = np.arange(e - a)
            valid[a:e] = True
    nb = np.where(valid, (pos + 1) // max(wl.c, 1), 0)
    return nb, valid


def _fwd_source_hash():
    h = hashlib.sha256()
    for path in FWD_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per forward call from the committed PMC summary, or None if the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_fwd_source_sha256_16") != _fwd_source_hash():
        return None
    return t


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

    if args.sweep:
        sweep(args)
        return
    if args.peaks:
        peaks()
        return
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = irb.load_library()
    sptr = irb._stream(dev)
    stream = torch.cuda.current_stream(dev)
    P = irb._ptr
    C = irb._check

    t0 = time.time()
    parts = ("attn", "bwd", "idx") if wl.latent else (("route", "attn", "bwd") if wl.backward else ("route", "attn"))
    x = synth.make_inputs(wl, parts=parts)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    act = ("kI", "qI", "q", "k", "v", "kv", "dO")
    d = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(dev).to(dt if k in act else torch.from_numpy(v).dtype))
         for k, v in x.items() if isinstance(v, np.ndarray) and k != "cu_seqlens"}
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).to(dev)
    gen_s = time.time() - t0
    S, B = wl.S, wl.B
    R = args.route_groups
    if R != 1 and (wl.latent or R != wl.Hkv or wl.H_idx % R):
        print(f"--route-groups must be 1 or the KV head count ({wl.Hkv}), dividing the index heads", file=sys.stderr)
        sys.exit(2)
    G_lead = (R,) if R > 1 else ()
    stages = {}          # name -> list of (start, end) events per timed step

    # ---------------------------------------------------------------- buffers (the step allocates nothing)
    if wl.latent:
        Hkv, Dqk, Dv = 1, wl.D, wl.Dv
        W = wl.latent_width
        L = W
        scale = wl.softmax_scale
        idx = d["idx"].reshape(S, W)
        routes = torch.empty((1, S, W), dtype=torch.int32, device=dev)
        lens = torch.empty((1, S), dtype=torch.int32, device=dev)
        bad = torch.zeros(1, dtype=torch.int32, device=dev)
        q = d["q"][None]
        k = d["kv"][None]
        v = k[..., :Dv]
        dO = d["dO"][None]
    else:
        Hkv, Dqk, Dv = wl.Hkv, wl.D, wl.Dv
        scale = 1.0 / math.sqrt(wl.D)
        c, topk, window = wl.c, wl.topk, wl.window
        L = irb.route_width(topk, c, window)
        nb_blocks = S // c
        # the fused call covers every row: the score kernel skips rows that see at most topk
        # blocks and the selection takes all their visible blocks without reading scores
        q0 = 0
        fused_ws = torch.empty(max(int(lib.irb_route_topk_fused_groups_workspace_size(
            B, S, c, wl.D_idx, topk, q0, S, R)), 4), dtype=torch.uint8, device=dev)
        sel = torch.empty(G_lead + (B, S, topk), dtype=torch.int32, device=dev)
        cnt = torch.empty(G_lead + (B, S), dtype=torch.int32, device=dev)
        routes = torch.empty(G_lead + (B, S, L), dtype=torch.int32, device=dev)
        lens = torch.empty(G_lead + (B, S), dtype=torch.int32, device=dev)
        sel_g, cnt_g = sel.view(R, B, S, topk), cnt.view(R, B, S)
        routes_g, lens_g = routes.view(R, B, S, L), lens.view(R, B, S)
        kc = torch.empty((B, nb_blocks, wl.D_idx), dtype=torch.float32, device=dev)
        cu_blocks = None if cu is None else torch.empty(cu.numel(), dtype=torch.int32, device=dev)
        lay = irb.make_layout(B, S, cu, None)
        qprep = torch.empty_like(d["qI"])
        sel_bitmap = torch.empty(G_lead + (B, S, (nb_blocks + 31) // 32), dtype=torch.int32, device=dev)
        q, k, v = d["q"], d["k"], d["v"]
        dO = d.get("dO")
    Hq = wl.Hq
    out = torch.empty((B, S, Hq, Dv), dtype=dt, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    # training steps keep o in FP32 as well where the backward reads its row
    # statistic off it (the library says where; elsewhere it forms it itself)
    keep_o32 = wl.backward and bool(lib.irb_sparse_gqa_attention_bwd_reads_out_f32(
        B, S, S, L, Hq, Hkv, Dqk, Dv, irb._dtype_code(q), R))
    out32 = torch.empty((B, S, Hq, Dv), dtype=torch.float32, device=dev) if keep_o32 else None
    strides = irb._strides9(q, k, v)
    fwd_ws_n = int(lib.irb_sparse_gqa_attention_fwd_workspace_size(B, S, S, L, Hq, Hkv, Dqk, Dv, irb._dtype_code(q), R))
    fwd_ws = torch.empty(max(fwd_ws_n, 16), dtype=torch.uint8, device=dev)
    backward = wl.backward
    if backward:
        rbq, rbk = 1, 16
        nkt, nqt = -(-S // rbk), -(-S // rbq)
        # grouped routes: R * B route rows, one reverse list per (group, row, key tile)
        rev_counts = torch.empty((R * B, nkt), dtype=torch.int32, device=dev)
        rev_idx = torch.empty((R * B, nkt, nqt), dtype=torch.int32, device=dev)
        lists_ws = torch.empty(max(int(lib.irb_build_block_lists_workspace_size(R * B, S, S, rbq, rbk)), 4),
                               dtype=torch.uint8, device=dev)
        full_counts, part_counts = torch.empty_like(rev_counts), torch.empty_like(rev_counts)
        full_idx, part_idx = torch.empty_like(rev_idx), torch.empty_like(rev_idx)
        split_ws = torch.empty(max(int(lib.irb_split_full_blocks_workspace_size(R * B, S, S, rbq, rbk)), 4),
                               dtype=torch.uint8, device=dev)
        dq = torch.empty((B, S, Hq, Dqk), dtype=dt, device=dev)
        dk = torch.empty((B, S, Hkv, Dqk), dtype=dt, device=dev)
        dv = dk if wl.latent else torch.empty((B, S, Hkv, Dv), dtype=dt, device=dev)
        dropped = torch.zeros(1, dtype=torch.int64, device=dev)
        bwd_ws = torch.empty(max(int(lib.irb_sparse_gqa_attention_bwd_workspace_size(
            B, S, S, L, Hq, Hkv, Dqk, Dv, irb._dtype_code(q), R)), 4), dtype=torch.uint8, device=dev)

    # cold-cache mode: a 512 MiB write on the same stream before each timed call
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev) if args.cold else None

    def timed(name, fn, record):
        if record:
            if flush is not None:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            stages.setdefault(name, []).append((e0, e1))
        else:
            fn()

    # ---------------------------------------------------------------- the step
    def route_step(rec):
        if wl.latent:
            timed("compact", lambda: C(lib.irb_compact_routes(P(idx), S, W, S, P(routes), P(lens), P(bad), sptr)), rec)
            return
        timed("compress", lambda: C(lib.irb_compress_keys(
            irb.ctypes.byref(lay), c, P(d["kI"]), irb._dtype_code(d["kI"]), d["kI"].stride(0), d["kI"].stride(1),
            wl.D_idx, P(d["gamma"]), 1e-5, P(d["freqs"]), d["freqs"].shape[-1], P(kc), P(cu_blocks), sptr)), rec)
        if R == 1:
            # raw index queries: RMSNorm (gain gamma) and RoPE at each token, fused into the scoring
            timed("score_select", lambda: C(lib.irb_route_topk_fused_raw(
                irb.ctypes.byref(lay), P(d["qI"]), irb._dtype_code(d["qI"]), wl.H_idx, wl.D_idx, P(d["gamma"]), 1e-5,
                P(d["freqs"]), d["freqs"].shape[-1], P(d["w"]), P(kc), P(cu_blocks), c, 1.0 / math.sqrt(wl.D_idx),
                topk, q0, S, P(sel), P(cnt), P(fused_ws), fused_ws.numel(), sptr)), rec)
        else:
            # index heads [H_idx] read as [R, H_idx / R]: one score row and selection per KV group
            # (the workload's index queries taken as prepared)
            timed("score_select", lambda: C(lib.irb_route_topk_fused_groups(
                irb.ctypes.byref(lay), P(d["qI"]), irb._dtype_code(d["qI"]), R, wl.H_idx // R, wl.D_idx, P(d["w"]),
                P(kc), P(cu_blocks), c, 1.0 / math.sqrt(wl.D_idx), topk, q0, S, P(sel), P(cnt), P(fused_ws),
                fused_ws.numel(), sptr)), rec)
        timed("expand", lambda: [C(lib.irb_expand_and_compact_routes(
            irb.ctypes.byref(lay), P(sel_g[g]), P(cnt_g[g]), topk, c, window, P(cu_blocks), L, P(routes_g[g]),
            P(lens_g[g]), sptr)) for g in range(R)], rec)

    def attn_step(rec):
        timed("attn_fwd", lambda: C(lib.irb_sparse_gqa_attention_fwd(
            P(q), P(k), P(v), irb._dtype_code(q), strides, P(routes), P(lens), R, B, S, S, L, Hq, Hkv, Dqk, Dv,
            scale, P(out), P(lse), P(out32) if out32 is not None else None, P(fwd_ws) if fwd_ws_n > 0 else None,
            fwd_ws_n, sptr)), rec)
        if backward:
            timed("reverse_lists", lambda: C(lib.irb_build_block_lists(
                P(routes), P(lens), R * B, S, S, L, rbq, rbk, 1, P(rev_counts), P(rev_idx), nqt, P(lists_ws),
                lists_ws.numel(), sptr)), rec)
            timed("attn_bwd", lambda: C(lib.irb_sparse_gqa_attention_bwd(
                P(q), P(k), P(v), irb._dtype_code(q), strides, P(out32), P(dO), P(lse), P(routes), P(lens), R,
                P(rev_counts), P(rev_idx), rbq, rbk, nqt, B, S, S, L, Hq, Hkv, Dqk, Dv, scale, P(dq), P(dk), P(dv),
                P(bwd_ws), bwd_ws.numel(), P(dropped), sptr)), rec)

    # Step-5 CSA calls (S=8192 workload only): regions = the complete groups of c
    # tokens, compression logits drawn N(0,1) in bf16 by a seeded device
    # generator, the fused route call's score tile materialised once (untimed)
    csa = (not wl.latent) and wl.name == "s8192" and R == 1
    if csa:
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed + 77)
        csa_logits = torch.randn((B, S, wl.D_idx), generator=gen, device=dev).to(torch.bfloat16)
        csa_src = (torch.arange(nb_blocks, device=dev, dtype=torch.int32)[:, None] * c
                   + torch.arange(c, device=dev, dtype=torch.int32)[None, :]).expand(B, nb_blocks, c).contiguous()
        csa_valid = torch.ones((B, nb_blocks, c), dtype=torch.uint8, device=dev)
        csa_pk = torch.empty((B, nb_blocks, c, wl.D_idx), dtype=torch.bfloat16, device=dev)
        csa_pz = torch.empty_like(csa_pk)
        csa_sum = torch.empty((B, nb_blocks, wl.D_idx), dtype=torch.bfloat16, device=dev)
        csa_q = torch.empty_like(d["qI"])
        csa_scores = torch.empty((B, S, nb_blocks), dtype=torch.float32, device=dev)
        csa_ids = torch.empty((B, S, topk + 1), dtype=torch.int32, device=dev)
        csa_cnt = torch.empty((B, S), dtype=torch.int32, device=dev)
        csa_ws = torch.empty(max(int(lib.irb_select_regions_csa_workspace_size(B, S, topk, 0)), 16), dtype=torch.uint8,
                             device=dev)

    def aux_step(rec):
        """Calls timed beside the step, outside it: nothing in the step reads their outputs."""
        if wl.latent:
            return
        if csa:
            timed("csa_gather_payload", lambda: C(lib.irb_gather_region_payload(
                P(d["kI"]), P(csa_logits), 1, B, S, wl.D_idx, P(csa_src), P(csa_valid), nb_blocks, c, P(csa_pk),
                P(csa_pz), sptr)), rec)
            timed("csa_summarize", lambda: C(lib.irb_summarize_region_payload(
                P(csa_pk), P(csa_pz), 1, P(csa_valid), B, nb_blocks, c, wl.D_idx, P(csa_sum), sptr)), rec)
            timed("csa_round_queries", lambda: C(lib.irb_round_e4m3(
                P(d["qI"]), 1, d["qI"].numel(), P(csa_q), sptr)), rec)
            timed("csa_select", lambda: C(lib.irb_select_regions_csa(
                irb.ctypes.byref(lay), P(csa_scores), nb_blocks, 0, S, None, c, topk, P(csa_ids), P(csa_cnt),
                P(csa_ws), csa_ws.numel(), sptr)), rec)
        # index-query preparation materialised by its own call (the step fuses it into scoring)
        timed("prepare_queries", lambda: C(lib.irb_prepare_index_queries(
            P(d["qI"]), irb._dtype_code(d["qI"]), B * S, wl.H_idx, wl.D_idx, P(d["gamma"]), 1e-5, P(d["freqs"]),
            d["freqs"].shape[-1], P(qprep), sptr)), rec)
        # route bitmap of the selection (membership words per query)
        timed("region_bitmap", lambda: C(lib.irb_pack_region_bitmap(
            P(sel), R * B * S, topk, nb_blocks, P(sel_bitmap), sptr)), rec)
        if backward:
            # full/partial split of the reverse lists
            timed("split_full_blocks", lambda: C(lib.irb_split_full_blocks(
                P(routes), P(lens), R * B, S, S, L, rbq, rbk, 1, P(rev_counts), P(rev_idx), nqt, P(full_counts),
                P(full_idx), P(part_counts), P(part_idx), P(split_ws), split_ws.numel(), sptr)), rec)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        route_step(False)
        attn_step(False)
    torch.cuda.synchronize()

    step_ev = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        route_step(True)
        attn_step(True)
        e1.record(stream)
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # the auxiliary calls, after the timed steps (same number of repetitions)
    if csa:
        C(lib.irb_indexer_score_tile(irb.ctypes.byref(lay), P(d["qI"]), 1, wl.H_idx, wl.D_idx, P(d["w"]), P(kc), None, c,
                                     0.0, 0, S, 0, nb_blocks, P(csa_scores), nb_blocks, sptr))
    for _ in range(2):
        aux_step(False)
    for _ in range(args.steps):
        aux_step(True)
    torch.cuda.synchronize()
    ms = {name: float(np.mean([a.elapsed_time(b) for a, b in evs])) for name, evs in stages.items()}
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in step_ev]))

    # ---------------------------------------------------------------- algorithmic work per call
    # selected pairs: (route group, query, key) entries; each serves the
    # Hq / R query heads (and Hkv / R KV heads) that read that group's routes
    lens_h = lens.cpu().numpy().astype(np.int64).reshape(R, -1)
    pairs = int(lens_h.sum())
    valid_q = int((lens_h > 0).any(axis=0).sum())
    fwd_flop = 2.0 * (Dqk + Dv) * (Hq // R) * pairs
    gathered = 2.0 * (Dqk + Dv) * (Hkv // R) * pairs if not wl.latent else 2.0 * Dqk * pairs
    work = {"attn_fwd": ("mfma", fwd_flop)}
    if backward:
        work["attn_bwd"] = ("mfma", 2.0 * (3 * Dqk + 2 * Dv) * (Hq // R) * pairs)
        # routes read + counts and the index matrix written: the call's output is
        # [rows, width] with -1 after each count, every entry of it written
        work["reverse_lists"] = ("hbm", 4.0 * L * R * B * S + 4.0 * rev_counts.numel() + 4.0 * rev_idx.numel())
        # listed entries read and written once (plus counts), and (one-query tiles) every
        # route read once to mark the key tiles it holds completely, one bit each
        entries = float(rev_counts.sum().item())
        work["split_full_blocks"] = ("hbm", 8.0 * entries + 12.0 * rev_counts.numel()
                                     + 4.0 * float(lens.sum().item()) + float(split_ws.numel()))
    if wl.latent:
        work["compact"] = ("hbm", (8.0 * W + 4.0) * S)
        route_ms = ms["compact"]
    else:
        nb_t, valid_t = _layout_counts(wl, S, x["cu_seqlens"])
        sparse_pairs = float(np.sum(np.where(nb_t > topk, nb_t, 0)))
        work["prepare_queries"] = ("hbm", 2.0 * B * S * wl.H_idx * wl.D_idx * d["qI"].element_size()
                                   + 4.0 * B * S * d["freqs"].shape[-1])
        work["compress"] = ("hbm", B * S * wl.D_idx * (2 if dt == torch.bfloat16 else 4)
                            + B * nb_blocks * (4 * wl.D_idx + 4 * d["freqs"].shape[-1]))
        # per route group: its own bitmap, selection and expansion; the
        # scoring work is the same in total (each group scores H_idx / R heads)
        work["region_bitmap"] = ("hbm", R * B * S * (4.0 * topk + 4.0 * ((nb_blocks + 31) // 32)))
        if csa:
            slots = float(B * nb_blocks * c)
            # gather: keys and logits rows read and written, plus the source ids and valid flags
            work["csa_gather_payload"] = ("hbm", slots * (4 * 2 * wl.D_idx + 5))
            work["csa_summarize"] = ("hbm", slots * (2 * 2 * wl.D_idx + 1) + 2.0 * B * nb_blocks * wl.D_idx)
            work["csa_round_queries"] = ("hbm", 4.0 * d["qI"].numel())
            hist = np.where(valid_t, np.arange(S) // c, 0)
            work["csa_select"] = ("hbm", 4.0 * float(np.sum(np.where(hist > topk, hist, 0)))
                                  + 4.0 * (topk + 1) * S * B + 4.0 * S * B)
        work["score_select"] = ("mfma", 2.0 * wl.H_idx * wl.D_idx * sparse_pairs)
        work["expand"] = ("hbm", R * float(np.sum(valid_t)) * (4 * topk + 4 * L + 4))
        route_ms = sum(ms[n] for n in ("compress", "score_select", "expand") if n in ms)
    stage_out, aux_out = {}, {}
    aux_names = ("prepare_queries", "region_bitmap", "split_full_blocks", "csa_gather_payload", "csa_summarize",
                 "csa_round_queries", "csa_select")
    for name, t in ms.items():
        bound, amount = work[name]
        if bound == "mfma":
            ach = amount / (t / 1e3) / 1e12
            (aux_out if name in aux_names else stage_out)[name] = {"ms": round(t, 4), "bound": "mfma", "achieved": round(ach, 3), "unit": "TFLOP/s",
                               "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 5),
                               "work": amount}
        else:
            ach = amount / (t / 1e3) / 1e9
            (aux_out if name in aux_names else stage_out)[name] = {"ms": round(t, 4), "bound": "hbm", "achieved": round(ach, 1), "unit": "GB/s",
                               "peak": HBM_PEAK_GBS, "frac": round(ach / HBM_PEAK_GBS, 5), "work": amount}
    if args.cold:
        # the flushes sit between the step's calls: the step is its calls' sum
        step_ms = sum(v["ms"] for v in stage_out.values())
    fwd_s = ms["attn_fwd"] / 1e3
    tflops = fwd_flop / fwd_s / 1e12
    qps = valid_q / (route_ms / 1e3)

    traffic = None
    # the counter record is of the default (warm) run
    tr = _traffic() if wl.name == "s8192" and R == 1 and not args.cold else None
    if tr is not None:
        traffic = tr["hbm_bytes_per_call"]

    result = {
        "metric": "sparse-attn fwd TFLOP/s (selected pairs) + routed queries/s, S=8192",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "routed_queries_per_s": round(qps, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_route": round(route_ms, 4),
        "ms_attn_fwd": round(ms["attn_fwd"], 4),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "cache": "cold" if args.cold else "warm",
        "config": {
            "workload": wl.name, "description": wl.description, "B": B, "S": S, "Hq": Hq, "Hkv": Hkv,
            "Dqk": Dqk, "Dv": Dv, "route_width": L, "selected_pairs": pairs, "valid_queries": valid_q,
            "backward_in_step": backward, "route_groups": R,
            **({} if wl.latent else {"H_idx": wl.H_idx, "D_idx": wl.D_idx, "c": wl.c, "topk": wl.topk,
                                     "window": wl.window}),
        },
        "roofline": {
            "kernel": "sparse_gqa_attention_fwd (route_bits_kernel + attn_fwd_tile_kernel)",
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 5),
            "traffic": traffic,
            "algorithmic_flop_per_launch": fwd_flop,
            "avg_launch_ms": round(ms["attn_fwd"], 5),
            "gathered_GBps": round(gathered / fwd_s / 1e9, 1),
        },
        "stages": stage_out,
        "aux_calls_outside_step": aux_out,
        "input_gen_s": round(gen_s, 2),
    }
    if backward:
        result["bwd_dropped_hits"] = int(dropped.item())
    if not args.no_cpu_baseline and wl.name == "s8192" and R == 1:
        result["cpu_baseline"], check = cpu_baseline(wl, x, args.cpu_sample_rows, sel.cpu().numpy())
        result["near_tie_rows"] = check["near_tie_rows"]
        result["route_check"] = check
    print(json.dumps(result), flush=True)


def peaks():
    """Achievable ceilings beside the published peaks: a bf16 GEMM through the
    vendor BLAS (torch.matmul, 8192^3, FP32 accumulate) and a 4 GiB device copy,
    each the median of 10 HIP-event timings after 3 warm-ups."""
    import numpy as np
    import torch

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)

    def med(fn, n=10):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts]))

    N = 8192
    a = torch.randn((N, N), generator=gen, device=dev).to(torch.bfloat16)
    b = torch.randn((N, N), generator=gen, device=dev).to(torch.bfloat16)
    c = torch.empty((N, N), dtype=torch.bfloat16, device=dev)
    ms_gemm = med(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    n = (4 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms_copy = med(lambda: dst.copy_(src))
    gemm_tflops = 2.0 * N ** 3 / (ms_gemm / 1e3) / 1e12
    copy_gbs = 2.0 * n * 4 / (ms_copy / 1e3) / 1e9
    print(json.dumps({"peaks": "achievable ceilings", "bf16_gemm_8192": {"ms": round(ms_gemm, 4),
                      "TFLOPs": round(gemm_tflops, 1), "frac_of_published": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
                      "device_copy_4GiB": {"ms": round(ms_copy, 4), "GBps_read_plus_write": round(copy_gbs, 1),
                                           "frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 4)}}), flush=True)


def sweep(args):
    """HBM rate of key compression and index-query preparation against sequence length.

    Synthetic bf16 inputs of the S=8192 workload's shapes (D_idx = 128, c = 4,
    16 index heads, full-width rotary table), drawn by a seeded torch
    generator on the device; each size is timed with HIP events on the
    kernels' stream (5 warm-ups, median of 20).  Bytes are the algorithmic
    ones of the step's stages.
    """
    import numpy as np
    import torch

    import indexer_routed_block_amd as irb

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = irb.load_library()
    sptr = irb._stream(dev)
    stream = torch.cuda.current_stream(dev)
    P, C = irb._ptr, irb._check
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    D, c, H = 128, 4, 16
    rows = []
    for S in (8192, 32768, 131072, 524288, 2097152):
        kI = torch.randn((1, S, D), generator=gen, device=dev).to(torch.bfloat16)
        qI = torch.randn((1, S, H, D), generator=gen, device=dev).to(torch.bfloat16)
        freqs = torch.rand((1, S, D), generator=gen, device=dev)
        gamma = torch.ones(D, dtype=torch.float32, device=dev)
        kc = torch.empty((1, S // c, D), dtype=torch.float32, device=dev)
        qout = torch.empty_like(qI)
        lay = irb.make_layout(1, S, None, None)
        calls = {
            "compress": (lambda: C(lib.irb_compress_keys(irb.ctypes.byref(lay), c, P(kI), 1, kI.stride(0), kI.stride(1), D,
                                                         P(gamma), 1e-5, P(freqs), D, P(kc), None, sptr)),
                         S * D * 2 + (S // c) * (4 * D + 4 * D)),
            "prepare_queries": (lambda: C(lib.irb_prepare_index_queries(P(qI), 1, S, H, D, P(gamma), 1e-5, P(freqs), D,
                                                                        P(qout), sptr)),
                                2 * S * H * D * 2 + 4 * S * D),
        }
        entry = {"S": S}
        for name, (fn, nbytes) in calls.items():
            for _ in range(5):
                fn()
            ts = []
            for _ in range(20):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
            gbs = nbytes / (ms / 1e3) / 1e9
            entry[name] = {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(gbs, 1),
                           "frac": round(gbs / HBM_PEAK_GBS, 4)}
        rows.append(entry)
        del kI, qI, freqs, kc, qout
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "token-streaming kernels vs sequence length", "peak_GBps": HBM_PEAK_GBS,
                      "rows": rows}), flush=True)


def cpu_baseline(wl, x, n_rows, gpu_sel):
    """The FP64 oracle on a bounded sample: n_rows query rows spread over the sequence.

    Route pipeline (compress all blocks, then score / select / expand the
    sampled rows) and the attention forward of the same rows, each timed
    with perf_counter on this host's cores.

    The route side starts from the raw index queries: the oracle's FP64
    RMSNorm + RoPE, rounded to bf16 (nearest even) as the fused GPU call
    rounds its FP32 result, then scores and top-k.

    Also returns, untimed, the selection check of every query row: the
    oracle's scores and top-k for all rows against the selection the timed
    GPU steps produced (``gpu_sel`` [B, S, topk]); rows whose k-th and
    (k+1)-th oracle scores lie within 1e-4 relative are counted as near ties.
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
    # the raw index queries' RMSNorm + RoPE, stored in bf16 as the GPU stores them
    f, e = np.frexp(oracle.prepare_index_queries(x["qI"], x["gamma"], x["freqs"], 1e-5))
    qp = np.ldexp(np.rint(f * 256.0), e - 8)
    sel = np.full((1, S, wl.topk), -1, dtype=np.int32)
    cnt = np.zeros((1, S), dtype=np.int32)
    for t in rows:
        s = oracle.indexer_scores(qp, x["w"], kc, wl.c, q0=int(t), q1=int(t) + 1)
        st, ct = oracle.select_topk(s, wl.c, wl.topk, q0=int(t), S=S)
        sel[0, t], cnt[0, t] = st[0, 0], ct[0, 0]
    routes, _ = oracle.expand_routes(sel, cnt, wl.c, wl.window, wl.topk, rows=[(0, int(t)) for t in rows])
    route_s = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.attention_fwd(x["q"], x["k"], x["v"], routes, rows=[(0, int(t)) for t in rows])
    attn_s = time.perf_counter() - t1
    pairs = int((routes[0, rows] >= 0).sum())
    flop = 2.0 * (wl.D + wl.Dv) * wl.Hq * pairs
    t2 = time.perf_counter()
    s_all = oracle.indexer_scores(qp, x["w"], kc, wl.c)
    sel_all, _ = oracle.select_topk(s_all, wl.c, wl.topk)
    ties = oracle.near_tie_rows(s_all, wl.c, wl.topk)
    gpu_sel = np.asarray(gpu_sel)
    differ = ~np.all(gpu_sel == sel_all, axis=-1)
    # a differing row must still be a correct top-k: within the FP32 scoring
    # bound plus the score change of the prepared elements whose bf16 rounding
    # the FP32 preparation may take either way
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
    from gpu_util import SCORE_ERR, prep_term_bound, score_bound
    q64 = np.asarray(x["qI"], dtype=np.float64)
    p64 = oracle.prepare_index_queries(q64, x["gamma"], x["freqs"], 1e-5)
    E = prep_term_bound(q64, x["gamma"], x["freqs"], x["freqs"].shape[-1])
    f1, e1 = np.frexp(p64 + E)
    f0, e0 = np.frexp(p64 - E)
    amb = np.ldexp(np.rint(f1 * 256.0), e1 - 8) - np.ldexp(np.rint(f0 * 256.0), e0 - 8)
    scale = 1.0 / math.sqrt(wl.D_idx)
    outside = 0
    for t in np.argwhere(differ[0])[:, 0]:
        s = s_all[0, t]
        n = int(np.isfinite(s).sum())
        M = score_bound(qp[:, t:t + 1], x["w"][:, t:t + 1], kc, scale)[0, 0, :n]
        A = scale * (np.abs(x["w"][0, t]) @ (np.abs(amb[0, t]) @ np.abs(kc[0, :n]).T))
        slack = SCORE_ERR * M + A
        inside = np.zeros(n, dtype=bool)
        inside[gpu_sel[0, t][gpu_sel[0, t] >= 0]] = True
        if inside.all():
            continue
        if np.min(s[:n][inside] + slack[inside]) < np.max(s[:n][~inside] - slack[~inside]):
            outside += 1
    check = {"rows": int(ties.size), "near_tie_rows": int(ties.sum()), "rows_differing": int(differ.sum()),
             "non_tie_rows_differing": int((differ & ~ties).sum()),
             "rows_differing_outside_bound": outside,
             "oracle_s": round(time.perf_counter() - t2, 2)}
    return {"value": round(flop / attn_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} query rows (evenly spaced from S/4 to S-1) of the {wl.name} workload; FP64 NumPy; "
                      f"attention fwd {attn_s:.2f} s, route pipeline {route_s:.2f} s "
                      f"({n_rows / route_s:.1f} routed queries/s incl. full key compression)"}, check


if __name__ == "__main__":
    main()
