"""GPU parity of per-KV-group routes against the FP64 oracle, through the C ABI:
grouped index scores, grouped fused selection + expansion (+ route bitmaps),
and sparse attention forward / backward whose KV groups read their own routes.

Grouped index queries are the workload's own seeded index queries with the
head axis split into groups (H_idx = groups x heads per group).  Tolerances:
scores within 1e-3 of the magnitude bound sum |w| sum |q k|
(gpu_util.score_bound), as for shared routes; selections, routes and
lengths bit-exact wherever the GPU selects what the oracle selects, and
every other row a correct top-k under the FP32 scoring bound (see
_check_grouped_selection); attention as gpu_util.attn_tol_check.
"""
import math

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import SCORE_ERR, act_dtype, attn_tol_check, banner, check_selection, host, score_bound, to_dev

pytestmark = pytest.mark.gpu


def _layout(name, S):
    if name == "single":
        return None, None, 1
    if name == "rows":
        return None, np.array([S, S // 3 + 5, 0], dtype=np.int32), 3
    rng = np.random.default_rng(S)
    cu, _ = synth.varlen_documents(rng, S, min_len=16, max_len=max(32, S // 3), max_pad=min(511, S // 8))
    return cu, None, 1


def _grouped_inputs(wl_name, S, layout, R):
    wl = synth.WORKLOADS[wl_name]
    cu, rl, B = _layout(layout, S)
    x = synth.make_inputs(wl, parts=("route",), S=S, B=B, cu_seqlens=cu, row_lens=rl)
    H = wl.H_idx // R
    x["qI"] = np.ascontiguousarray(x["qI"].reshape(B, S, R, H, wl.D_idx))
    x["w"] = np.ascontiguousarray(x["w"].reshape(B, S, R, H))
    dt = act_dtype(wl.dtype)
    d = dict(kI=to_dev(x["kI"], dt), qI=to_dev(x["qI"], dt), w=to_dev(x["w"]), gamma=to_dev(x["gamma"]),
             freqs=to_dev(x["freqs"]), cu=to_dev(x["cu_seqlens"]), rl=to_dev(x["row_lens"]))
    return wl, x, d


@pytest.mark.parametrize("wl_name,S,layout,R", [("s8192", 2048, "single", 4), ("varlen", 4096, "packed", 4),
                                                ("long", 2048, "single", 8), ("s8192", 1500, "rows", 2),
                                                ("long", 2048, "single", 4), ("long", 1024, "single", 2),
                                                ("tiny", 512, "single", 1)])
def test_grouped_score_tile(wl_name, S, layout, R):
    """Groups of 4 and 8 heads over 16 or 32 index heads run in one launch
    (s8192: 4x4, 2x8; long: 8x4, 4x8); long with 2 groups of 16 heads and
    the tiny workload take the per-group loop."""
    banner(f"grouped score {wl_name} S={S} {layout} groups={R}")
    wl, x, d = _grouped_inputs(wl_name, S, layout, R)
    kc_h, cub = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, x["cu_seqlens"], x["row_lens"])
    kc, cu_blocks = to_dev(kc_h.astype(np.float32)), to_dev(cub)
    scale = 1.0 / math.sqrt(wl.D_idx)
    nb = S // wl.c
    for (q0, q1, j0, j1) in [(0, S, 0, nb), (S // 3 + 1, S - 7, nb // 5 + 3, nb - 2)]:
        got = host(irb.indexer_score_tile(d["qI"], d["w"], kc, wl.c, q0, q1, j0, j1, scale, cu_blocks, d["cu"], d["rl"]))
        ref = oracle.indexer_scores_grouped(x["qI"], x["w"], kc_h, wl.c, scale, x["cu_seqlens"], x["row_lens"],
                                            q0, q1)[..., j0:j1]
        assert got.shape == ref.shape
        assert np.array_equal(np.isneginf(got), np.isneginf(ref))
        for g in range(R):
            M = score_bound(x["qI"][:, q0:q1, g], x["w"][:, q0:q1, g], kc_h[:, j0:j1], scale)
            fin = np.isfinite(ref[g])
            err = np.abs(got[g][fin] - ref[g][fin])
            assert np.all(err <= SCORE_ERR * M[fin] + 1e-30), f"group {g}: max rel-to-M {np.max(err / M[fin]):.2e}"


def _oracle_grouped_routes(wl, x, topk):
    kc, _ = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, x["cu_seqlens"], x["row_lens"])
    s = oracle.indexer_scores_grouped(x["qI"], x["w"], kc, wl.c, None, x["cu_seqlens"], x["row_lens"])
    out = dict(sel=[], cnt=[], routes=[], lens=[], ties=[])
    for g in range(s.shape[0]):
        sel, cnt = oracle.select_topk(s[g], wl.c, topk, x["cu_seqlens"], x["row_lens"])
        routes, lens = oracle.expand_routes(sel, cnt, wl.c, wl.window, topk, x["cu_seqlens"], x["row_lens"])
        out["sel"].append(sel); out["cnt"].append(cnt); out["routes"].append(routes); out["lens"].append(lens)
        out["ties"].append(oracle.near_tie_rows(s[g], wl.c, topk, x["cu_seqlens"], x["row_lens"]))
    out = {k: np.stack(v) for k, v in out.items()}
    out["kc"] = kc
    return out


def _check_grouped_selection(wl, x, topk, r, ref):
    """Every row of every group: bit-exact where the selection equals the
    oracle's, else a correct top-k under the FP32 scoring bound whose routes
    expand the GPU's own selection (gpu_util.check_selection)."""
    got = {k: host(r[k]) for k in ("sel", "cnt", "routes", "lens")}
    check_selection(wl, x, topk, got, ref, ref["kc"], grouped=True)


@pytest.mark.parametrize("wl_name,S,layout,R", [("s8192", 2048, "single", 4), ("varlen", 4096, "packed", 4),
                                                ("long", 4096, "single", 8), ("s8192", 1500, "rows", 2),
                                                ("long", 4096, "single", 4)])
def test_grouped_route_pipeline(wl_name, S, layout, R):
    """compress -> grouped fused score/select -> per-group expand (+ bitmaps); bit-exact outside near ties."""
    banner(f"grouped pipeline {wl_name} S={S} {layout} groups={R}")
    wl, x, d = _grouped_inputs(wl_name, S, layout, R)
    topk = min(wl.topk, max(4, S // wl.c // 4))
    r = irb.route(d["kI"], d["qI"], d["w"], d["gamma"], d["freqs"], wl.c, topk, wl.window, cu_seqlens=d["cu"],
                  row_lens=d["rl"])
    ref = _oracle_grouped_routes(wl, x, topk)
    _check_grouped_selection(wl, x, topk, r, ref)
    # the groups really select differently (a shared or swapped group would not)
    if R > 1:
        assert not np.array_equal(ref["sel"][0], ref["sel"][1])
    # membership words of a grouped selection, [R, B, S, words] (the oracle's
    # selection on both sides)
    nb = S // wl.c
    bm = host(irb.pack_region_bitmap(to_dev(ref["sel"].astype(np.int32)), nb))
    np.testing.assert_array_equal(bm, oracle.pack_region_bitmap(ref["sel"], nb))


def _group_random_routes(seed, R, B, S, width, empty=()):
    rng = np.random.default_rng(seed)
    rs, ls = [], []
    for g in range(R):
        ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.25)
        r, n, _ = oracle.compact_routes(ids, S)
        for (gg, b, t) in empty:
            if gg == g:
                r[b, t] = -1
                n[b, t] = 0
        rs.append(r)
        ls.append(n)
    return np.stack(rs), np.stack(ls)


def _check_lse(got, want, dtype):
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    tol = 1e-3 if dtype == torch.bfloat16 else 1e-4
    assert np.max(np.abs(got[fin] - want[fin]), initial=0.0) <= tol


def _fwd_bwd(q_h, k_h, v_h, dO_h, routes, lens, scale, dt, rev_bq=None):
    q, k, v = to_dev(q_h, dt), to_dev(k_h, dt), to_dev(v_h, dt)
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, scale)
    ro, rlse = oracle.attention_fwd_grouped(q_h, k_h, v_h, routes, scale)
    attn_tol_check(host(o), ro, dt, "o")
    _check_lse(host(lse), rlse, dt)
    if rev_bq is None:
        return
    S_k = k_h.shape[1]
    rc, ri = irb.build_block_lists(r_d, l_d, S_k, rev_bq, 16, reverse=True)
    dO = to_dev(dO_h, dt)
    dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, rev_bq, 16, scale)
    rdq, rdk, rdv = oracle.attention_bwd_grouped(q_h, k_h, v_h, routes, dO_h, scale)
    attn_tol_check(host(dq), rdq, dt, "dq")
    attn_tol_check(host(dk), rdk, dt, "dk")
    attn_tol_check(host(dv), rdv, dt, "dv")


def test_grouped_pipeline_routes_attention_fwd():
    """S=8192 recipe at S=2048: 4 KV groups, each with its own selection + window
    routes (dense early tiles on the tile kernel, later ones gathered)."""
    banner("grouped attn fwd s8192 recipe S=2048 pipeline routes")
    wl, x, _ = _grouped_inputs("s8192", 2048, "single", 4)
    topk = min(wl.topk, max(4, 2048 // wl.c // 4))
    ref = _oracle_grouped_routes(wl, x, topk)
    a = synth.make_inputs(wl, parts=("attn",), S=2048)
    _fwd_bwd(a["q"], a["k"], a["v"], None, ref["routes"], ref["lens"], 1.0 / math.sqrt(wl.D), torch.bfloat16)


@pytest.mark.parametrize("S,width,rev_bq", [(1024, 160, 1), (333, 70, 16), (700, 700, 1)])
def test_grouped_bf16_random_routes_fwd_bwd(S, width, rev_bq):
    """GQA 32/4 bf16, D=128: random per-group routes (the widest are dense
    enough for the tile kernel), empty rows in one group only."""
    banner(f"grouped attn bf16 S={S} width={width} rev_bq={rev_bq}")
    wl = synth.WORKLOADS["varlen"]
    a = synth.make_inputs(wl, parts=("attn", "bwd"), S=S)
    routes, lens = _group_random_routes(S + 7, wl.Hkv, 1, S, width, empty=[(1, 0, 5), (3, 0, S - 1)])
    _fwd_bwd(a["q"], a["k"], a["v"], a["dO"], routes, lens, 1.0 / math.sqrt(wl.D), torch.bfloat16, rev_bq)


@pytest.mark.parametrize("Hq,Hkv,D,B", [(8, 2, 64, 2), (16, 4, 64, 1), (32, 2, 128, 1)])
def test_grouped_other_shapes_fwd_bwd(Hq, Hkv, D, B):
    """bf16 head groups of 4, 4 and 16 (every tile-kernel instantiation with
    per-group routes) with B > 1 rows."""
    banner(f"grouped attn bf16 Hq={Hq} Hkv={Hkv} D={D} B={B}")
    rng = np.random.default_rng(Hq * 100 + D)
    S = 300
    q = synth.to_bf16_values(rng.standard_normal((B, S, Hq, D)).astype(np.float32))
    k = synth.to_bf16_values(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    v = synth.to_bf16_values(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    dO = synth.to_bf16_values(rng.standard_normal((B, S, Hq, D)).astype(np.float32))
    routes, lens = _group_random_routes(Hq + D, Hkv, B, S, 200)
    _fwd_bwd(q, k, v, dO, routes, lens, 1.0 / math.sqrt(D), torch.bfloat16, 1)


def test_grouped_fp32_fwd_bwd():
    """FP32 inputs (split-precision gather path and the transposed-copy backward), two KV groups of 2 heads."""
    banner("grouped attn fp32 Hq=4 Hkv=2 D=64")
    rng = np.random.default_rng(91)
    B, S, Hq, Hkv, D = 1, 257, 4, 2, 64
    q = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    dO = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    routes, lens = _group_random_routes(92, Hkv, B, S, 40, empty=[(0, 0, 9)])
    _fwd_bwd(q, k, v, dO, routes, lens, 0.125, torch.float32, 3)


def test_identical_group_routes_match_shared_routes():
    """Grouped routes that repeat one route give the shared-route results bit for bit."""
    banner("grouped attn: identical groups vs shared")
    wl = synth.WORKLOADS["varlen"]
    S = 512
    a = synth.make_inputs(wl, parts=("attn", "bwd"), S=S)
    routes, lens = _group_random_routes(5, 1, 1, S, 120)
    q, k, v, dO = (to_dev(a[n], torch.bfloat16) for n in ("q", "k", "v", "dO"))
    r1, l1 = to_dev(routes[0]), to_dev(lens[0])
    rg = to_dev(np.ascontiguousarray(np.repeat(routes, wl.Hkv, axis=0)))
    lg = to_dev(np.ascontiguousarray(np.repeat(lens, wl.Hkv, axis=0)))
    o1, s1 = irb.sparse_gqa_attention_fwd(q, k, v, r1, l1)
    o2, s2 = irb.sparse_gqa_attention_fwd(q, k, v, rg, lg)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    g1 = irb.sparse_gqa_attention_bwd(q, k, v, o1, dO, s1, r1, l1, *irb.build_block_lists(r1, l1, S, 1, 16, True), 1)
    g2 = irb.sparse_gqa_attention_bwd(q, k, v, o2, dO, s2, rg, lg, *irb.build_block_lists(rg, lg, S, 1, 16, True), 1)
    for x1, x2 in zip(g1, g2):
        assert torch.equal(x1, x2)


def test_grouped_full_size_s8192():
    """S=8192 workload with its 16 index heads read as 4 groups (the bench's
    --route-groups 4 configuration): every row's selection and routes of every
    group outside near ties, then the forward on sampled rows of every head."""
    wl = synth.WORKLOADS["s8192"]
    S, R = wl.S, wl.Hkv
    banner(f"grouped full size s8192 S={S} groups={R}")
    wl, x, d = _grouped_inputs("s8192", S, "single", R)
    r = irb.route(d["kI"], d["qI"], d["w"], d["gamma"], d["freqs"], wl.c, wl.topk, wl.window)
    ref = _oracle_grouped_routes(wl, x, wl.topk)
    _check_grouped_selection(wl, x, wl.topk, r, ref)
    # forward over the oracle's grouped routes (both sides), checked on sampled rows
    ref_routes = np.ascontiguousarray(ref["routes"].astype(np.int32))
    ref_lens = np.ascontiguousarray(ref["lens"].astype(np.int32))
    a = synth.make_inputs(wl, parts=("attn",))
    q, k, v = (to_dev(a[n], torch.bfloat16) for n in ("q", "k", "v"))
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, to_dev(ref_routes), to_dev(ref_lens))
    rng = np.random.default_rng(8192)
    rows = sorted(set([0, 1, 2047, 2048, S - 1] + rng.integers(0, S, 43).tolist()))
    todo = [(0, int(t)) for t in rows]
    ro, rlse = oracle.attention_fwd_grouped(a["q"], a["k"], a["v"], ref_routes, 1.0 / math.sqrt(wl.D), rows=todo)
    attn_tol_check(host(o)[0, rows], ro[0, rows], torch.bfloat16, "o (sampled rows)")
    _check_lse(host(lse)[0][:, rows], rlse[0][:, rows], torch.bfloat16)
