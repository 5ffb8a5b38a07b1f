"""GPU parity at the workloads' full sizes, through the C ABI.

The FP64 oracle cannot evaluate every row at these sizes, so each test runs
the GPU path over the whole workload and checks

* every output the oracle produces cheaply at full size: compressed keys,
  the per-row selection count k_eff, the compaction of the latent index
  lists, and (S=8192) the whole route pipeline;
* sampled query rows and key tiles, which the oracle evaluates one by one;
* properties that hold at any size, over every row: routes ascending with a
  -1 suffix, ids causal and inside the query's document, the sliding window
  and the incomplete-group tail present; and exact gradient identities --
  per KV head, the sum over keys of dV equals the sum of dO over the head's
  query heads and non-empty queries, the sum over keys of dK is zero, and
  sum_t q_t . dq_t equals sum_k dK_k . k_k.

Attention routes for the packed and the 131072-token workloads come from a
random choice of k_eff visible blocks per query (uniform draws from
``synth``, turned into blocks and expanded by the oracle), because scoring
every block in FP64 would take hours at those sizes; the S=8192 workload
uses the oracle's full route pipeline.
"""
import functools
import math
import time

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import DEV, SCORE_ERR, act_dtype, attn_tol_check, banner, check_selection, host, score_bound, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BF16 = torch.bfloat16
ID_TOL = 2.0 ** -7      # identities: two bf16 half-ulps of the summed magnitudes


def _log(msg, t0):
    print(f"    {msg} [{time.time() - t0:.1f}s]", flush=True)


@functools.lru_cache(maxsize=None)
def _inputs(name, parts):
    return synth.make_inputs(synth.WORKLOADS[name], parts=parts)


@functools.lru_cache(maxsize=None)
def _info(name):
    wl = synth.WORKLOADS[name]
    cu = _inputs(name, ("layout",))["cu_seqlens"]
    docs = oracle.documents(1, wl.S, cu, None)
    return cu, oracle.token_info(docs, wl.S, wl.c)


@functools.lru_cache(maxsize=None)
def _oracle_pipeline(name):
    wl = synth.WORKLOADS[name]
    x = _inputs(name, ("route",))
    return oracle.route_pipeline(x["kI"], x["qI"], x["w"], x["gamma"], x["freqs"], wl.c, wl.topk, wl.window,
                                 cu_seqlens=x["cu_seqlens"])


@functools.lru_cache(maxsize=None)
def _attn_routes(name):
    """Token routes for the attention tests (see the module docstring)."""
    wl = synth.WORKLOADS[name]
    if name == "s8192":
        r = _oracle_pipeline(name)
        return r["routes"], r["lens"]
    cu, (valid, start, base, nb) = _info(name)
    u = _inputs(name, ("draws",))["draws"]
    slot = np.arange(wl.topk)
    nb3 = nb[..., None].astype(np.int64)
    keff = np.minimum(wl.topk, nb)
    # every visible block when there are at most topk of them, else uniform draws
    pick = np.minimum((u.astype(np.float64) * nb3).astype(np.int64), np.maximum(nb3 - 1, 0))
    local = np.where(nb3 <= wl.topk, slot, pick)
    sel = np.where(slot < keff[..., None], base[..., None] + local, -1).astype(np.int32)
    cnt = np.where(valid, keff, 0).astype(np.int32)
    return oracle.expand_routes(sel, cnt, wl.c, wl.window, wl.topk, cu_seqlens=cu)


def _row_ranges(name, width=8, n_rand=4):
    """Starts of 8-row query ranges: sequence ends, document starts/middles/ends,
    the padding tail, the first row that needs scoring, and random rows."""
    wl = synth.WORKLOADS[name]
    S = wl.S
    cu, _ = _info(name)
    starts = {0, S - width}
    if cu is None:
        f = irb.first_sparse_query(wl.c, wl.topk)
        starts |= {f - width // 2, S // 3, S // 2}
    else:
        lens = np.diff(cu)
        order = np.argsort(lens, kind="stable")
        for d in (order[0], order[len(order) // 2], order[-1]):
            a, e = int(cu[d]), int(cu[d + 1])
            starts |= {a, e - width, (a + e) // 2}
        starts.add(int(cu[-1]))
    rng = np.random.default_rng(wl.seed)
    starts |= set(int(s) for s in rng.integers(0, S - width, n_rand))
    return sorted({min(max(0, s), S - width) for s in starts})


def _sample_rows(name, n=48):
    rows = set()
    for s in _row_ranges(name):
        rows |= {s, s + 3, s + 7}
    rng = np.random.default_rng(synth.WORKLOADS[name].seed + 1)
    rows |= set(int(t) for t in rng.integers(0, synth.WORKLOADS[name].S, max(0, n - len(rows))))
    return sorted(rows)


def _check_route_invariants(name, routes_d, lens_d, sel_d=None, cnt_d=None):
    """Properties of every row of GPU routes (and selections) that hold at any size."""
    wl = synth.WORKLOADS[name]
    S, L = wl.S, routes_d.shape[-1]
    cu, (valid, start, base, nb) = _info(name)
    R, n = routes_d[0], lens_d[0].long()
    t = torch.arange(S, device=DEV)
    a = to_dev(start[0].astype(np.int64))
    v = to_dev(valid[0])
    ok = R >= 0
    assert torch.equal(ok.sum(1), n), "length != number of valid ids"
    assert torch.equal(ok, torch.arange(L, device=DEV)[None] < n[:, None]), "valid ids are not a prefix"
    assert not ((R[:, 1:] <= R[:, :-1]) & ok[:, 1:]).any(), "ids not strictly ascending"
    assert not (ok & ((R > t[:, None]) | (R < a[:, None]))).any(), "id outside [document start, t]"
    assert not (n[~v] != 0).any(), "padding query with a route"
    # the tail [a + nb*c, t] and the window [max(a, t-W+1), t] are both present
    lo = a + to_dev(nb[0].astype(np.int64)) * wl.c
    if wl.window > 0:
        lo = torch.minimum(lo, torch.maximum(a, t - wl.window + 1))
    have = (ok & (R >= lo[:, None])).sum(1)
    assert torch.equal(have[v], (t - lo + 1)[v]), "window or incomplete-group tail missing"
    if sel_d is not None:
        keff = np.where(valid, np.minimum(wl.topk, nb), 0)[0]
        np.testing.assert_array_equal(host(cnt_d)[0], keff)
        s, c_ = sel_d[0], cnt_d[0].long()
        used = torch.arange(wl.topk, device=DEV)[None] < c_[:, None]
        b0 = to_dev(base[0].astype(np.int64))
        b1 = b0 + to_dev(nb[0].astype(np.int64))
        assert not (used & ((s < b0[:, None]) | (s >= b1[:, None]))).any(), "selected block not visible"
        assert not ((s[:, 1:] <= s[:, :-1]) & used[:, 1:]).any(), "selected blocks not ascending"
        assert not (~used & (s != -1)).any(), "selection slots past k_eff are not -1"


@pytest.mark.parametrize("name", ["s8192", "varlen", "long"])
def test_route_pipeline_full_size(name):
    wl = synth.WORKLOADS[name]
    banner(f"full-size route pipeline {name} S={wl.S}")
    t0 = time.time()
    x = _inputs(name, ("route",))
    cu = x["cu_seqlens"]
    dt = act_dtype(wl.dtype)
    d = dict(kI=to_dev(x["kI"], dt), qI=to_dev(x["qI"], dt), w=to_dev(x["w"]), gamma=to_dev(x["gamma"]),
             freqs=to_dev(x["freqs"]), cu=to_dev(cu))
    _log("inputs", t0)
    r = irb.route(d["kI"], d["qI"], d["w"], d["gamma"], d["freqs"], wl.c, wl.topk, wl.window, cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    _log("gpu pipeline", t0)
    kc_ref, cub_ref = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, cu)
    np.testing.assert_allclose(host(r["kc"]), kc_ref, rtol=1e-5, atol=1e-5)
    if cub_ref is not None:
        np.testing.assert_array_equal(host(r["cu_blocks"]), cub_ref)
    _check_route_invariants(name, r["routes"], r["lens"], r["sel"], r["cnt"])
    _log("compress + invariants", t0)
    scale = 1.0 / math.sqrt(wl.D_idx)
    kc_d = to_dev(kc_ref.astype(np.float32))
    cub_d = to_dev(cub_ref)
    got_sel, got_routes, got_lens = host(r["sel"]), host(r["routes"]), host(r["lens"])
    got = {"sel": got_sel[None], "cnt": host(r["cnt"])[None], "routes": got_routes[None], "lens": got_lens[None]}
    if name == "s8192":
        # every row: bit-exact outside near ties, near-tie rows a valid top-k expanded exactly
        ref = _oracle_pipeline(name)
        want = {k: ref[k][None] for k in ("sel", "cnt", "routes", "lens")}
        want["ties"] = oracle.near_tie_rows(ref["scores"], wl.c, wl.topk)[None]
        n_ties, n_diff = check_selection(wl, x, wl.topk, got, want, kc_ref, grouped=False)
        print(f"    all {wl.S} rows: near-tie {n_ties}, differing {n_diff}")
    sel_ref = np.full((1, wl.S, wl.topk), -1, dtype=np.int32)
    cnt_ref = np.zeros((1, wl.S), dtype=np.int32)
    rows, n_ties = [], 0
    tie_rows = set()
    for s0 in _row_ranges(name):
        s1 = s0 + 8
        ref_s = oracle.indexer_scores(x["qI"], x["w"], kc_ref, wl.c, scale, cu, q0=s0, q1=s1)
        got_s = host(irb.indexer_score_tile(d["qI"], d["w"], kc_d, wl.c, s0, s1, 0, wl.S // wl.c, scale, cub_d,
                                            d["cu"]))
        assert np.array_equal(np.isneginf(got_s), np.isneginf(ref_s)), f"visibility differs in rows {s0}..{s1}"
        fin = np.isfinite(ref_s)
        M = score_bound(x["qI"][:, s0:s1], x["w"][:, s0:s1], kc_ref, scale)
        err = np.abs(got_s[fin] - ref_s[fin])
        assert np.all(err <= SCORE_ERR * M[fin] + 1e-30), f"scores rows {s0}..{s1}: max err/M {np.max(err / M[fin]):.2e}"
        st, ct = oracle.select_topk(ref_s, wl.c, wl.topk, cu, q0=s0, S=wl.S)
        sel_ref[0, s0:s1], cnt_ref[0, s0:s1] = st[0], ct[0]
        ties = oracle.near_tie_rows(ref_s, wl.c, wl.topk, cu, q0=s0, S=wl.S)[0]
        tie_rows |= {s0 + i for i in np.nonzero(ties)[0]}
        rows += list(range(s0, s1))
    rows = sorted(set(rows))
    routes_ref, lens_ref = oracle.expand_routes(sel_ref, cnt_ref, wl.c, wl.window, wl.topk, cu_seqlens=cu,
                                                rows=[(0, t) for t in rows])
    print(f"    sampled rows {len(rows)}, near-tie {len(tie_rows)}")
    # the sampled rows take the every-row check; the others carry the GPU's own values (compared to themselves)
    want = {k: v.copy() for k, v in got.items()}
    for key, arr in (("sel", sel_ref), ("cnt", cnt_ref), ("routes", routes_ref), ("lens", lens_ref)):
        want[key][0, 0, rows] = arr[0, rows]
    want["ties"] = np.zeros((1, 1, wl.S), dtype=bool)
    want["ties"][0, 0, sorted(tie_rows)] = True
    check_selection(wl, x, wl.topk, got, want, kc_ref, grouped=False)
    _log("sampled rows", t0)


def _fwd(name, x, routes, lens, o32=False):
    """The forward as the step runs it: training workloads also keep the FP32 output
    (the backward's Delta input), which the stored output must round to exactly."""
    wl = synth.WORKLOADS[name]
    q, k, v = (to_dev(x[n], BF16) for n in ("q", "k", "v"))
    r_d, l_d = to_dev(routes), to_dev(lens)
    if not o32:
        o, lse = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, 1.0 / math.sqrt(wl.D))
        return q, k, v, r_d, l_d, o, lse
    o, lse, out32 = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, 1.0 / math.sqrt(wl.D), out_f32=True)
    assert torch.equal(o, out32.to(BF16)), "o is not the rounding of the FP32 output"
    return q, k, v, r_d, l_d, o, lse, out32


def _check_fwd_rows(name, x, routes, lens, o, lse, rows):
    wl = synth.WORKLOADS[name]
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], routes, 1.0 / math.sqrt(wl.D),
                                    rows=[(0, t) for t in rows])
    attn_tol_check(host(o)[0, rows], ro[0, rows], BF16, f"o ({len(rows)} rows)")
    got_l, want_l = host(lse)[0][:, rows], rlse[0][:, rows]
    fin = np.isfinite(want_l)
    assert np.array_equal(np.isneginf(got_l), ~fin)
    assert np.max(np.abs(got_l[fin] - want_l[fin]), initial=0.0) <= 1e-3
    # every row: lse is -inf exactly where the route is empty, and o is zero there
    empty = to_dev(lens[0] == 0)
    assert torch.equal(torch.isneginf(lse[0]), empty[None].expand(wl.Hq, -1))
    assert not o[0][empty].any()


@pytest.mark.parametrize("name", ["s8192", "varlen", "long"])
def test_attention_fwd_full_size(name):
    wl = synth.WORKLOADS[name]
    banner(f"full-size attention fwd {name} S={wl.S}")
    t0 = time.time()
    routes, lens = _attn_routes(name)
    x = _inputs(name, ("attn",))
    _log(f"routes + inputs (pairs {int(lens.sum())})", t0)
    q, k, v, r_d, l_d, o, lse = _fwd(name, x, routes, lens)
    torch.cuda.synchronize()
    _log("gpu fwd", t0)
    # S=8192: every query row against the oracle; the longer workloads: sampled rows
    rows = list(range(wl.S)) if name == "s8192" else _sample_rows(name)
    _check_fwd_rows(name, x, routes, lens, o, lse, rows)
    _log(f"{len(rows)} rows", t0)


def _key_tiles(name):
    """16-key tiles whose gradients the oracle evaluates.

    One causal document: the last tile and the tile 2048 keys before the
    end (reached through the window and through selected blocks).  Packed
    documents: the last tile (padding), the middle of the sequence, and the
    second and last tiles of the longest document.  Tiles far from the end
    of a long document are reached by thousands of queries, too many to
    evaluate one by one in FP64.
    """
    wl = synth.WORKLOADS[name]
    S = wl.S
    tiles = {S // 16 - 1}
    cu, _ = _info(name)
    if cu is None:
        tiles.add((S - 2048) // 16)
    else:
        tiles.add((S // 2) // 16)
        d = int(np.argmax(np.diff(cu)))
        tiles.add((int(cu[d + 1]) - 1) // 16)
        tiles.add(int(cu[d]) // 16 + 1)
    return sorted(tiles)


def _identities(wl, x, q, k, dO, lens, dq, dk, dv, G):
    """Exact gradient identities over all keys (see the module docstring)."""
    S = wl.S
    f64 = torch.float64
    live = to_dev(lens[0] > 0)
    dO64 = dO[0].to(f64) * live[:, None, None]
    for name_, got, want, mag in (
        ("sum_k dV = sum dO", dv[0].to(f64).sum(0),
         dO64.reshape(S, wl.Hkv, G, wl.Dv).sum((0, 2)), dv[0].to(f64).abs().sum(0)),
        ("sum_k dK = 0", dk[0].to(f64).sum(0), torch.zeros_like(dk[0, 0], dtype=f64), dk[0].to(f64).abs().sum(0)),
    ):
        err = (got - want).abs()
        print(f"    {name_}: max err {float(err.max()):.3e}, bound {ID_TOL:.4f}*sum|.| min {float((ID_TOL * mag).min()):.3e}, "
              f"max err/sum|.| {float((err / mag.clamp_min(1e-30)).max()):.2e}")
        assert bool((err <= ID_TOL * mag + 1e-6).all()), name_
    qq = (q[0].to(f64) * dq[0].to(f64)).reshape(S, wl.Hkv, G, -1).sum(-1)
    kk = (dk[0].to(f64) * k[0].to(f64)).sum(-1)
    lhs, rhs = qq.sum((0, 2)), kk.sum(0)
    mag = qq.abs().sum((0, 2)) + kk.abs().sum(0)
    err = (lhs - rhs).abs()
    print(f"    sum_t q.dq = sum_k dK.k: err/sum|.| {float((err / mag).max()):.2e}")
    assert bool((err <= ID_TOL * mag).all()), "trace identity"


@pytest.mark.parametrize("name", ["varlen", "long"])
def test_attention_bwd_full_size(name):
    wl = synth.WORKLOADS[name]
    banner(f"full-size attention bwd {name} S={wl.S}")
    t0 = time.time()
    routes, lens = _attn_routes(name)
    x = _inputs(name, ("attn",))
    xb = _inputs(name, ("bwd",))
    S, G = wl.S, wl.Hq // wl.Hkv
    scale = 1.0 / math.sqrt(wl.D)
    _log("routes + inputs", t0)
    q, k, v, r_d, l_d, o, lse, o32 = _fwd(name, x, routes, lens, o32=True)
    rc, ri = irb.build_block_lists(r_d, l_d, S, 1, 16, reverse=True)
    dO = to_dev(xb["dO"], BF16)
    torch.cuda.synchronize()
    g0 = time.time()
    dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, 1, 16, scale, out_f32=o32)
    torch.cuda.synchronize()
    _log(f"gpu fwd + lists + bwd (bwd {time.time() - g0:.2f}s)", t0)
    tiles = _key_tiles(name)
    rc_ref, ri_ref = oracle.block_lists(routes, lens, S, 1, 16, reverse=True, rows=[(0, j) for j in tiles])
    rc_h, ri_h = host(rc), host(ri)
    for j in tiles:
        n = int(rc_ref[0, j])
        assert int(rc_h[0, j]) == n, f"reverse list count of key tile {j}"
        np.testing.assert_array_equal(ri_h[0, j, :n], ri_ref[0, j, :n])
    _log(f"reverse lists of tiles {tiles}", t0)
    rows = _sample_rows(name, 24)
    keys = [(0, 16 * j + i) for j in tiles for i in range(16) if 16 * j + i < S]
    rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], routes, xb["dO"], scale,
                                         rows=[(0, t) for t in rows], keys=keys)
    kid = [kk for _, kk in keys]
    attn_tol_check(host(dq)[0, rows], rdq[0, rows], BF16, f"dq ({len(rows)} rows)")
    attn_tol_check(host(dk)[0, kid], rdk[0, kid], BF16, f"dk ({len(kid)} keys)")
    attn_tol_check(host(dv)[0, kid], rdv[0, kid], BF16, f"dv ({len(kid)} keys)")
    _log("sampled rows and keys", t0)
    _identities(wl, x, q, k, dO, lens, dq, dk, dv, G)
    _log("identities", t0)


def test_latent_full_size():
    wl = synth.WORKLOADS["latent"]
    T, H, Dv = wl.S, wl.Hq, wl.Dv
    banner(f"full-size latent T={T} H={H} width={wl.latent_width}")
    t0 = time.time()
    x = _inputs("latent", ("attn", "bwd", "idx"))
    idx = x["idx"]
    routes, lens, bad = oracle.compact_routes(idx[:, 0, :], T)
    assert bad == 0
    _log("inputs + oracle compaction", t0)
    idx_d = to_dev(idx[:, 0, :])
    r_gpu, l_gpu, n_bad = irb.compact_routes(idx_d, T)
    assert int(n_bad.item()) == 0
    np.testing.assert_array_equal(host(r_gpu), routes)
    np.testing.assert_array_equal(host(l_gpu), lens)
    kv_d = to_dev(x["kv"], BF16)[None]
    q_d = to_dev(x["q"], BF16)[None]
    k_d, v_d = kv_d, kv_d[..., :Dv]
    r_d, l_d = to_dev(routes)[None], to_dev(lens)[None]
    o, lse, o32 = irb.sparse_gqa_attention_fwd(q_d, k_d, v_d, r_d, l_d, wl.softmax_scale, out_f32=True)
    assert torch.equal(o, o32.to(BF16)), "o is not the rounding of the FP32 output"
    rc, ri = irb.build_block_lists(r_d, l_d, T, 1, 16, reverse=True)
    dO = to_dev(x["dO"], BF16)[None]
    torch.cuda.synchronize()
    g0 = time.time()
    dq, dkv, _ = irb.sparse_gqa_attention_bwd(q_d, k_d, v_d, o, dO, lse, r_d, l_d, rc, ri, 1, 16,
                                              wl.softmax_scale, merged_kv=True, out_f32=o32)
    torch.cuda.synchronize()
    _log(f"compaction + fwd + lists + bwd (bwd {time.time() - g0:.2f}s)", t0)
    rows = _sample_rows_plain(T, wl.seed, 24)
    ro, rlse = oracle.latent_attention_fwd(x["q"][rows], x["kv"], idx[rows], wl.softmax_scale, dv=Dv)
    attn_tol_check(host(o)[0, rows], ro, BF16, f"latent o ({len(rows)} rows)")
    got_l = host(lse)[0][:, rows]
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isneginf(got_l), ~fin)
    assert np.max(np.abs(got_l[fin] - rlse[fin]), initial=0.0) <= 1e-3
    _log("fwd rows", t0)
    tiles = [T // 16 - 1, (3 * T // 4) // 16]
    keys = [16 * j + i for j in tiles for i in range(16)]
    rdq, rdkv = oracle.latent_attention_bwd(x["q"], x["kv"], idx, x["dO"], wl.softmax_scale, dv=Dv,
                                            rows=rows, keys=keys)
    attn_tol_check(host(dq)[0, rows], rdq[rows], BF16, f"latent dq ({len(rows)} rows)")
    attn_tol_check(host(dkv)[0, keys], rdkv[keys], BF16, f"latent dkv ({len(keys)} keys)")
    _log("bwd rows and keys", t0)
    # identities: dkv = dK + [dV, 0]; sum_k dK = 0 and sum_k dV = sum of dO over non-empty queries
    f64 = torch.float64
    live = to_dev(lens > 0)
    want = (dO[0].to(f64) * live[:, None, None]).sum((0, 1))
    tot = dkv[0, :, 0].to(f64).sum(0)
    mag = dkv[0, :, 0].to(f64).abs().sum(0)
    err = (tot - torch.cat([want, torch.zeros(wl.D - Dv, dtype=f64, device=DEV)])).abs()
    print(f"    latent sum_k dkv identity: max err/sum|.| {float((err / mag).max()):.2e}")
    assert bool((err <= ID_TOL * mag + 1e-6).all())


def _sample_rows_plain(T, seed, n):
    rng = np.random.default_rng(seed)
    rows = {0, 1, 7, T // 2, T - 2, T - 1}
    rows |= set(int(t) for t in rng.integers(0, T, n - len(rows)))
    return sorted(rows)


def _group_routes(name, R):
    """One route per KV group: the shared-route recipe with each group's own
    uniform block draws (seeded per group)."""
    wl = synth.WORKLOADS[name]
    cu, (valid, start, base, nb) = _info(name)
    slot = np.arange(wl.topk)
    nb3 = nb[..., None].astype(np.int64)
    keff = np.minimum(wl.topk, nb)
    cnt = np.where(valid, keff, 0).astype(np.int32)
    rs, ls = [], []
    for g in range(R):
        u = synth.make_inputs(wl, parts=("draws",), seed=wl.seed + 100 + g)["draws"]
        pick = np.minimum((u.astype(np.float64) * nb3).astype(np.int64), np.maximum(nb3 - 1, 0))
        local = np.where(nb3 <= wl.topk, slot, pick)
        sel = np.where(slot < keff[..., None], base[..., None] + local, -1).astype(np.int32)
        r, n = oracle.expand_routes(sel, cnt, wl.c, wl.window, wl.topk, cu_seqlens=cu)
        rs.append(r)
        ls.append(n)
    return np.stack(rs), np.stack(ls)


def test_grouped_attention_full_size_varlen():
    """Packed T=32768 training step with one route per KV group (4 groups):
    forward and dq on sampled rows of every head, dK/dV on sampled key tiles of
    every group, and per-group exact identities over every key."""
    name = "varlen"
    wl = synth.WORKLOADS[name]
    R, S, G = wl.Hkv, wl.S, wl.Hq // wl.Hkv
    banner(f"full-size grouped attention fwd+bwd {name} S={S} groups={R}")
    t0 = time.time()
    routes, lens = _group_routes(name, R)
    x = _inputs(name, ("attn",))
    xb = _inputs(name, ("bwd",))
    scale = 1.0 / math.sqrt(wl.D)
    _log("routes + inputs", t0)
    q, k, v = (to_dev(x[n], BF16) for n in ("q", "k", "v"))
    r_d, l_d = to_dev(routes), to_dev(lens)
    o, lse = irb.sparse_gqa_attention_fwd(q, k, v, r_d, l_d, scale)
    rc, ri = irb.build_block_lists(r_d, l_d, S, 1, 16, reverse=True)
    dO = to_dev(xb["dO"], BF16)
    dq, dk, dv = irb.sparse_gqa_attention_bwd(q, k, v, o, dO, lse, r_d, l_d, rc, ri, 1, 16, scale)
    torch.cuda.synchronize()
    _log("gpu fwd + lists + bwd", t0)
    rows = _sample_rows(name, 16)
    ro, rlse = oracle.attention_fwd_grouped(x["q"], x["k"], x["v"], routes, scale, rows=[(0, t) for t in rows])
    attn_tol_check(host(o)[0, rows], ro[0, rows], BF16, f"o ({len(rows)} rows)")
    got_l, want_l = host(lse)[0][:, rows], rlse[0][:, rows]
    fin = np.isfinite(want_l)
    assert np.array_equal(np.isneginf(got_l), ~fin)
    assert np.max(np.abs(got_l[fin] - want_l[fin]), initial=0.0) <= 1e-3
    tiles = [S // 16 - 1, (S // 2) // 16]
    keys = [(0, 16 * j + i) for j in tiles for i in range(16) if 16 * j + i < S]
    rdq, rdk, rdv = oracle.attention_bwd_grouped(x["q"], x["k"], x["v"], routes, xb["dO"], scale,
                                                 rows=[(0, t) for t in rows], keys=keys)
    kid = [kk for _, kk in keys]
    attn_tol_check(host(dq)[0, rows], rdq[0, rows], BF16, f"dq ({len(rows)} rows)")
    attn_tol_check(host(dk)[0, kid], rdk[0, kid], BF16, f"dk ({len(kid)} keys)")
    attn_tol_check(host(dv)[0, kid], rdv[0, kid], BF16, f"dv ({len(kid)} keys)")
    _log("sampled rows and keys", t0)
    # per KV head g (its own route's non-empty queries): sum_k dV = sum of dO over the group's heads,
    # sum_k dK = 0, and sum_t q.dq = sum_k dK.k
    f64 = torch.float64
    for g in range(R):
        live = to_dev(lens[g, 0] > 0)
        hs = slice(g * G, (g + 1) * G)
        want = (dO[0, :, hs].to(f64) * live[:, None, None]).sum((0, 1))
        dvg, dkg = dv[0, :, g].to(f64), dk[0, :, g].to(f64)
        assert bool(((dvg.sum(0) - want).abs() <= ID_TOL * dvg.abs().sum(0) + 1e-6).all()), f"sum dV, group {g}"
        assert bool((dkg.sum(0).abs() <= ID_TOL * dkg.abs().sum(0) + 1e-6).all()), f"sum dK, group {g}"
        qq = (q[0, :, hs].to(f64) * dq[0, :, hs].to(f64)).sum()
        kk = (dkg * k[0, :, g].to(f64)).sum()
        mag = (q[0, :, hs].to(f64) * dq[0, :, hs].to(f64)).abs().sum() + (dkg * k[0, :, g].to(f64)).abs().sum()
        assert bool((qq - kk).abs() <= ID_TOL * mag), f"trace identity, group {g}"
    _log("identities", t0)
