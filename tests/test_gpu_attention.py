"""GPU parity of sparse GQA attention forward/backward against the FP64 oracle, through the C ABI.

Tolerances: bf16 outputs and gradients mean-abs <= 5e-3 and per element
|err| <= 2e-2 + 2^-7 |ref| (see gpu_util.attn_tol_check; FP32 accumulation);
fp32 inputs max-abs <= 1e-4; lse within 1e-3 (bf16) / 1e-4 (fp32) absolute.
"""
import math
import types

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import DEV, act_dtype, attn_tol_check, banner, host, to_dev

pytestmark = pytest.mark.gpu


def _random_routes(seed, B, S, width, empty_rows=()):
    rng = np.random.default_rng(seed)
    ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.25)
    routes, lens, _ = oracle.compact_routes(ids, S)
    for (b, t) in empty_rows:
        routes[b, t] = -1
        lens[b, t] = 0
    return routes, lens


def _pipeline_routes(wl_name, S):
    wl = synth.WORKLOADS[wl_name]
    x = synth.make_inputs(wl, parts=("route",), S=S)
    topk = min(wl.topk, max(4, S // wl.c // 4))
    r = oracle.route_pipeline(x["kI"], x["qI"], x["w"], x["gamma"], x["freqs"], wl.c, topk, wl.window)
    return r["routes"], r["lens"]


def _qkv(wl_name, S, B=1, seed=None):
    wl = synth.WORKLOADS[wl_name]
    x = synth.make_inputs(wl, parts=("attn", "bwd"), S=S, B=B, seed=seed)
    return wl, x


def _check_lse(got, want, dtype):
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    tol = 1e-3 if dtype == torch.bfloat16 else 1e-4
    assert np.max(np.abs(got[fin] - want[fin]), initial=0.0) <= tol


def _run_fwd_bwd(wl, x, routes, lens, scale, do_bwd, q_view=None, rev_bq=1):
    dt = act_dtype(wl.dtype)
    q = to_dev(x["q"], dt) if q_view is None else q_view
    k = to_dev(x["k"], dt)
    v = to_dev(x["v"], dt)
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse, o32 = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, scale, out_f32=True)
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], routes, scale)
    attn_tol_check(host(o), ro, dt, "o")
    _check_lse(host(lse), rlse, dt)
    # the stored output is the FP32 output rounded once
    assert torch.equal(o, o32.to(o.dtype)), "o is not the rounding of the FP32 output"
    attn_tol_check(host(o32), ro, torch.float32 if dt == torch.float32 else dt, "o (fp32)")
    if not do_bwd:
        return
    S = x["q"].shape[1]
    rc, ri = irb.build_block_lists(r_d, l_d, S, rev_bq, 16, reverse=True)
    dO = to_dev(x["dO"], dt)
    rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], routes, x["dO"], scale)
    # Delta formed from the routes, then read off the forward's FP32 output
    for fo in (None, o32):
        dropped = torch.full((1,), -1, dtype=torch.int64, device=DEV)
        dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, rev_bq, 16, scale,
                                                  dropped_hits=dropped, out_f32=fo)
        assert int(dropped.item()) == 0, "reverse lists of the same routes dropped key-side hits"
        tag = "" if fo is None else " (Delta from the FP32 output)"
        attn_tol_check(host(dq), rdq, dt, "dq" + tag)
        attn_tol_check(host(dk), rdk, dt, "dk" + tag)
        attn_tol_check(host(dv), rdv, dt, "dv" + tag)


def test_tiny_fp32_pipeline_routes_fwd_bwd():
    banner("attn tiny fp32 S=512")
    wl, x = _qkv("tiny", 512)
    routes, lens = _pipeline_routes("tiny", 512)
    _run_fwd_bwd(wl, x, routes, lens, 1.0 / math.sqrt(wl.D), True)


@pytest.mark.parametrize("S,width,rev_bq", [(1024, 160, 1), (333, 70, 1), (1024, 160, 16), (333, 70, 3),
                                            (1024, 100, 1)])
def test_gqa_bf16_random_routes_fwd_bwd(S, width, rev_bq):
    """rev_bq > 1: reverse lists of query tiles, whose queries the backward
    searches for hits; rev_bq = 1: every listed query is a hit.  Routes at
    least 0.12 S wide (160 of 1024, 70 of 333) take every query tile in the
    query-tile launch, sparse tiles gathered there; narrower ones (100 of
    1024) leave the sparse tiles to the per-query gather launch."""
    banner(f"attn gqa bf16 S={S} width={width} rev_bq={rev_bq}")
    wl, x = _qkv("varlen", S)
    routes, lens = _random_routes(S, 1, S, width, empty_rows=[(0, 5), (0, S - 1)])
    _run_fwd_bwd(wl, x, routes, lens, 1.0 / math.sqrt(wl.D), True, rev_bq=rev_bq)


def test_gqa_bf16_window_routes_fwd():
    banner("attn s8192-recipe bf16 S=2048 pipeline routes")
    wl, x = _qkv("s8192", 2048)
    routes, lens = _pipeline_routes("s8192", 2048)
    _run_fwd_bwd(wl, x, routes, lens, 1.0 / math.sqrt(wl.D), False)


def test_gqa_bf16_batched_and_strided_q():
    banner("attn bf16 B=2 strided q")
    wl, x = _qkv("varlen", 256, B=2)
    routes, lens = _random_routes(7, 2, 256, 48, empty_rows=[(1, 0)])
    big = torch.zeros((2, 256, wl.Hq + 3, wl.D), dtype=torch.bfloat16, device=DEV)
    big[:, :, 1:1 + wl.Hq] = to_dev(x["q"], torch.bfloat16)
    qv = big[:, :, 1:1 + wl.Hq]
    assert not qv.is_contiguous()
    _run_fwd_bwd(wl, x, routes, lens, 0.11, True, q_view=qv)


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 4, 64), (16, 1, 64), (16, 2, 64), (8, 2, 128), (32, 2, 128), (32, 1, 128),
                                     (32, 1, 64)])
def test_gqa_bf16_head_groups_and_widths_fwd_bwd(Hq, Hkv, D):
    """Every (group size, head width) the query-tile and key-tile kernels are built for (G = 4, 8, 16; D = 64, 128),
    and G = 32 (one query per 32-row key-side batch; per-query forward and dQ).  The routes (96 of at most 300
    keys) overlap enough that most 64-key groups run in shared batches."""
    banner(f"attn bf16 Hq={Hq} Hkv={Hkv} D={D} S=300")
    rng = np.random.default_rng(1000 + 7 * Hq + 3 * Hkv + D)
    S = 300

    def nrm(*shape):
        return synth.to_bf16_values(rng.standard_normal(shape).astype(np.float32))

    x = {"q": nrm(1, S, Hq, D), "k": nrm(1, S, Hkv, D), "v": nrm(1, S, Hkv, D), "dO": nrm(1, S, Hq, D)}
    routes, lens = _random_routes(S + D + Hq, 1, S, 96, empty_rows=[(0, 7)])
    _run_fwd_bwd(types.SimpleNamespace(dtype="bf16"), x, routes, lens, 1.0 / math.sqrt(D), True)


@pytest.mark.parametrize("Hq,Hkv,D,S,width,rev_bq", [(8, 2, 128, 700, 200, 1), (4, 1, 64, 600, 300, 4)])
def test_fp32_head_widths_fwd_bwd(Hq, Hkv, D, S, width, rev_bq):
    """FP32 inputs at both head widths, routes wide enough that a key tile's
    reverse list holds several rounds of 256 query candidates (the key side
    splits them across a workgroup's four waves), with per-query and 4-query
    reverse tiles."""
    banner(f"attn fp32 Hq={Hq} Hkv={Hkv} D={D} S={S} width={width} rev_bq={rev_bq}")
    rng = np.random.default_rng(2000 + S + D)

    def nrm(*shape):
        return rng.standard_normal(shape).astype(np.float32)

    x = {"q": nrm(1, S, Hq, D), "k": nrm(1, S, Hkv, D), "v": nrm(1, S, Hkv, D), "dO": nrm(1, S, Hq, D)}
    routes, lens = _random_routes(S + width, 1, S, width, empty_rows=[(0, 3)])
    _run_fwd_bwd(types.SimpleNamespace(dtype="fp32"), x, routes, lens, 1.0 / math.sqrt(D), True, rev_bq=rev_bq)


@pytest.mark.parametrize("Hq,shared", [(16, False), (32, False), (16, True)])
def test_bf16_wide_heads_fwd_bwd(Hq, shared):
    """D = 576 / Dv = 512 outside the latent kernels' head count: the general
    forward; on the backward the per-tile key side (16 query heads) or the
    wide hit-list key side (32), with separate K and V, or one shared tensor
    (V its first 512 columns) whose merged gradient is dK + [dV, 0]."""
    banner(f"attn bf16 D=576/512 Hq={Hq} shared={shared}")
    rng = np.random.default_rng(576 + Hq + int(shared))
    S, Hkv, D, DV, width = 160, 1, 576, 512, 48

    def nrm(*shape):
        return synth.to_bf16_values(rng.standard_normal(shape).astype(np.float32))

    q, dO = nrm(1, S, Hq, D), nrm(1, S, Hq, DV)
    if shared:
        kv = nrm(1, S, Hkv, D)
        k, v = kv, np.ascontiguousarray(kv[..., :DV])
    else:
        k, v = nrm(1, S, Hkv, D), nrm(1, S, Hkv, DV)
    routes, lens = _random_routes(S + Hq, 1, S, width, empty_rows=[(0, 9)])
    scale = 1.0 / math.sqrt(D)
    dt = torch.bfloat16
    q_d, dO_d = to_dev(q, dt), to_dev(dO, dt)
    if shared:
        kv_d = to_dev(kv, dt)
        k_d, v_d = kv_d, kv_d[..., :DV]
    else:
        k_d, v_d = to_dev(k, dt), to_dev(v, dt)
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse = irb.sparse_gqa_attention_fwd(q_d, k_d, v_d, r_d, l_d, scale)
    ro, rlse = oracle.attention_fwd(q, k, v, routes, scale)
    attn_tol_check(host(o), ro, dt, "o")
    _check_lse(host(lse), rlse, dt)
    rc, ri = irb.build_block_lists(r_d, l_d, S, 1, 16, reverse=True)
    rdq, rdk, rdv = oracle.attention_bwd(q, k, v, routes, dO, scale)
    dropped = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    dq, dk, dv = irb.sparse_gqa_attention_bwd(q_d, k_d, v_d, o, dO_d, lse, r_d, l_d, rc, ri, 1, 16, scale,
                                              dropped_hits=dropped, merged_kv=shared)
    assert int(dropped.item()) == 0
    attn_tol_check(host(dq), rdq, dt, "dq")
    if shared:
        assert dv.data_ptr() == dk.data_ptr()
        rdkv = rdk.copy()
        rdkv[..., :DV] += rdv
        attn_tol_check(host(dk), rdkv, dt, "dkv (merged)")
    else:
        attn_tol_check(host(dk), rdk, dt, "dk")
        attn_tol_check(host(dv), rdv, dt, "dv")


@pytest.mark.parametrize("use_ws", [True, False])
def test_gqa_bf16_long_routes_fwd(use_ws):
    """Route rows past one round of the key-membership pass's loads (over 2560
    entries) and past several 512-entry staging chunks of the query-tile
    kernel's own mask building (without the workspace); G = 4 at D = 128 runs
    its mask segments at 128 key tiles, so 144 key tiles make two."""
    banner(f"attn bf16 long routes S=4608 G=4 D=128 workspace={use_ws}")
    rng = np.random.default_rng(4241)
    S, Hq, Hkv, D = 4608, 8, 2, 128

    def nrm(*shape):
        return synth.to_bf16_values(rng.standard_normal(shape).astype(np.float32))

    x = {"q": nrm(1, S, Hq, D), "k": nrm(1, S, Hkv, D), "v": nrm(1, S, Hkv, D)}
    ids = synth.random_routes(np.random.default_rng(4243), 1, S, 4400, causal=True, frac_invalid=0.25,
                              duplicates=False)
    routes, lens, _ = oracle.compact_routes(ids, S)
    assert int(lens.max()) > 2560
    dt = torch.bfloat16
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    scale = 1.0 / math.sqrt(D)
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, to_dev(routes), to_dev(lens), scale, use_workspace=use_ws)
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], routes, scale)
    attn_tol_check(host(o), ro, dt, "o")
    _check_lse(host(lse), rlse, dt)


@pytest.mark.parametrize("S_q,S_k,width,Hq,Hkv,D", [(300, 1000, 160, 16, 4, 128), (5, 4096, 2048, 32, 4, 128),
                                                    (77, 600, 64, 8, 2, 64)])
def test_gqa_bf16_fewer_queries_than_keys_fwd_bwd(S_q, S_k, width, Hq, Hkv, D):
    """Query and key counts differ (the calls take both): routes draw distinct
    keys from the whole key range, ascending, -1 after each row's length;
    wide rows take the query-tile kernel with its tiles partly past S_q, the
    narrowest the per-query gather.  The backward runs on reverse lists over
    the S_k keys, with Delta formed from the routes and from the FP32 output."""
    banner(f"attn bf16 S_q={S_q} S_k={S_k} width={width} Hq={Hq} Hkv={Hkv} D={D}")
    rng = np.random.default_rng(S_q * 7 + S_k)

    def nrm(*shape):
        return synth.to_bf16_values(rng.standard_normal(shape).astype(np.float32))

    x = {"q": nrm(1, S_q, Hq, D), "k": nrm(1, S_k, Hkv, D), "v": nrm(1, S_k, Hkv, D), "dO": nrm(1, S_q, Hq, D)}
    routes = np.full((1, S_q, width), -1, dtype=np.int32)
    lens = np.zeros((1, S_q), dtype=np.int32)
    for t in range(S_q):
        n = int(rng.integers(1, width + 1)) if t % 5 else width
        routes[0, t, :n] = np.sort(rng.choice(S_k, n, replace=False))
        lens[0, t] = n
    dt = torch.bfloat16
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    scale = 1.0 / math.sqrt(D)
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse, o32 = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, scale, out_f32=True)
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], routes, scale)
    attn_tol_check(host(o), ro, dt, "o")
    _check_lse(host(lse), rlse, dt)
    rc, ri = irb.build_block_lists(r_d, l_d, S_k, 1, 16, reverse=True)
    dO = to_dev(x["dO"], dt)
    rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], routes, x["dO"], scale)
    for fo in (None, o32):
        dropped = torch.full((1,), -1, dtype=torch.int64, device=DEV)
        dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, 1, 16, scale,
                                                  dropped_hits=dropped, out_f32=fo)
        assert int(dropped.item()) == 0
        tag = "" if fo is None else " (Delta from the FP32 output)"
        attn_tol_check(host(dq), rdq, dt, "dq" + tag)
        attn_tol_check(host(dk), rdk, dt, "dk" + tag)
        attn_tol_check(host(dv), rdv, dt, "dv" + tag)


def test_gqa_bf16_all_routes_empty_fwd_bwd():
    """No query routes to any key: o = 0 and lse = -inf for every row, empty
    reverse lists, and zero gradients (with and without the FP32 output)."""
    banner("attn bf16 all routes empty S=300")
    S, Hq, Hkv, D = 300, 32, 4, 128
    rng = np.random.default_rng(300)
    dt = torch.bfloat16
    q, k, v, dO = (to_dev(synth.to_bf16_values(rng.standard_normal(sh).astype(np.float32)), dt)
                   for sh in ((1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)))
    r_d = to_dev(np.full((1, S, 64), -1, dtype=np.int32))
    l_d = to_dev(np.zeros((1, S), dtype=np.int32))
    o, lse, o32 = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, out_f32=True)
    assert not torch.any(o != 0) and not torch.any(o32 != 0)
    assert torch.all(torch.isneginf(lse))
    rc, ri = irb.build_block_lists(r_d, l_d, S, 1, 16, reverse=True)
    assert not torch.any(rc != 0) and torch.all(ri == -1)
    for fo in (None, o32):
        dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, 1, 16, out_f32=fo)
        for g in (dq, dk, dv):
            assert not torch.any(g != 0)


@pytest.mark.parametrize("T,width", [(512, 256), (300, 64)])
def test_latent_shared_kv_fwd_bwd(T, width):
    banner(f"attn latent T={T} width={width}")
    wl = synth.WORKLOADS["latent"]
    x = synth.make_inputs(wl, parts=("attn", "bwd"), S=T)
    rng = np.random.default_rng(T)
    idx = synth.latent_indices(rng, T, width)
    routes, lens, _ = oracle.compact_routes(idx[:, 0, :], T)
    kv_d = to_dev(x["kv"], torch.bfloat16)[None]                      # [1, T, 1, 576]
    q_d = to_dev(x["q"], torch.bfloat16)[None]
    k_d, v_d = kv_d, kv_d[..., :wl.Dv]
    r_d, l_d = to_dev(routes)[None], to_dev(lens)[None]
    o, lse, o32 = irb.sparse_gqa_attention_fwd(q_d, k_d, v_d, r_d, l_d, wl.softmax_scale, out_f32=True)
    ro, rlse = oracle.latent_attention_fwd(x["q"], x["kv"], idx, wl.softmax_scale, dv=wl.Dv)
    attn_tol_check(host(o)[0], ro, torch.bfloat16, "latent o")
    _check_lse(host(lse)[0], rlse, torch.bfloat16)
    assert torch.equal(o, o32.to(torch.bfloat16)), "o is not the rounding of the FP32 output"
    rc, ri = irb.build_block_lists(r_d, l_d, T, 1, 16, reverse=True)
    dO = to_dev(x["dO"], torch.bfloat16)[None]
    rdq, rdkv = oracle.latent_attention_bwd(x["q"], x["kv"], idx, x["dO"], wl.softmax_scale, dv=wl.Dv)
    for fo in (None, o32):
        dq, dkv, dv_alias = irb.sparse_gqa_attention_bwd(q_d, k_d, v_d, o, dO, lse, r_d, l_d, rc, ri, 1, 16,
                                                         wl.softmax_scale, merged_kv=True, out_f32=fo)
        assert dv_alias.data_ptr() == dkv.data_ptr()
        tag = "" if fo is None else " (Delta from the FP32 output)"
        attn_tol_check(host(dq)[0], rdq, torch.bfloat16, "latent dq" + tag)
        attn_tol_check(host(dkv)[0], rdkv, torch.bfloat16, "latent dkv" + tag)


def test_backward_with_coarse_reverse_tiles():
    """Reverse lists at 16-query granularity give the same gradients as per-query lists."""
    banner("attn bwd coarse reverse lists")
    wl, x = _qkv("varlen", 400)
    routes, lens = _random_routes(11, 1, 400, 64)
    dt = torch.bfloat16
    q, k, v = (to_dev(x[n], dt) for n in ("q", "k", "v"))
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d)
    dO = to_dev(x["dO"], dt)
    a = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, *irb.build_block_lists(r_d, l_d, 400, 1, 16, True), 1)
    b = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, *irb.build_block_lists(r_d, l_d, 400, 16, 16, True), 16)
    for u, w_ in zip(a, b):
        assert torch.equal(u, w_)


def test_backward_counts_hits_past_the_workspace():
    """Reverse lists that do not belong to the routes (every key tile listing
    every query) give more key-side hit entries than the workspace holds: the
    extra ones are dropped and counted, and dq (query side) is unaffected."""
    banner("attn bwd stale reverse lists: dropped-hit counter")
    S, width = 256, 8
    wl, x = _qkv("varlen", S)
    routes, lens = _random_routes(5, 1, S, width)
    dt = torch.bfloat16
    q, k, v = (to_dev(x[n], dt) for n in ("q", "k", "v"))
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d)
    dO = to_dev(x["dO"], dt)
    nkt = S // 16
    rc = torch.full((1, nkt), S, dtype=torch.int32, device=DEV)
    ri = torch.arange(S, dtype=torch.int32, device=DEV).repeat(1, nkt, 1).contiguous()
    dropped = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, 1, dropped_hits=dropped)
    # capacity: S query rows x min(L, key tiles) entries; the lists hold S x key tiles
    want = S * nkt - S * min(width, nkt)
    assert int(dropped.item()) == want
    good_rc, good_ri = irb.build_block_lists(r_d, l_d, S, 1, 16, reverse=True)
    dq2, _, _ = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, good_rc, good_ri, 1)
    assert torch.equal(dq, dq2)
