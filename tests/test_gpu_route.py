"""GPU parity of the route pipeline (compress, score, select, expand, compact, block lists)
against the FP64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import indexer_routed_block_amd as irb
import oracle
import synth
from gpu_util import DEV, SCORE_ERR, act_dtype, banner, check_selection, host, score_bound as _score_bound, to_dev

pytestmark = pytest.mark.gpu


def _layout_case(name, S):
    """(cu_seqlens, row_lens, B) for a named layout at length S."""
    if name == "single":
        return None, None, 1
    if name == "rows":
        return None, np.array([S, S // 3 + 5, 0], dtype=np.int32), 3
    if name == "packed":
        rng = np.random.default_rng(S)
        cu, pad = synth.varlen_documents(rng, S, min_len=16, max_len=max(32, S // 3), max_pad=min(511, S // 8))
        return cu, None, 1
    raise ValueError(name)


def _inputs(wl_name, S, layout):
    wl = synth.WORKLOADS[wl_name]
    cu, rl, B = _layout_case(layout, S)
    x = synth.make_inputs(wl, parts=("route",), S=S, B=B, cu_seqlens=cu, row_lens=rl)
    return wl, x


def _dev_inputs(wl, x):
    dt = act_dtype(wl.dtype)
    return dict(kI=to_dev(x["kI"], dt), qI=to_dev(x["qI"], dt), w=to_dev(x["w"]), gamma=to_dev(x["gamma"]),
                freqs=to_dev(x["freqs"]), cu=to_dev(x["cu_seqlens"]), rl=to_dev(x["row_lens"]))


CASES = [("tiny", 512, "single"), ("tiny", 200, "rows"), ("s8192", 2048, "single"), ("varlen", 4096, "packed"),
         ("long", 2048, "single"), ("s8192", 1500, "rows")]


@pytest.mark.parametrize("wl_name,S,layout", CASES)
def test_compress_keys(wl_name, S, layout):
    banner(f"compress {wl_name} S={S} {layout}")
    wl, x = _inputs(wl_name, S, layout)
    d = _dev_inputs(wl, x)
    kc, cu_blocks = irb.compress_keys(d["kI"], d["gamma"], d["freqs"], wl.c, 1e-5, d["cu"], d["rl"])
    ref, ref_cub = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, x["cu_seqlens"], x["row_lens"])
    got = host(kc)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    if ref_cub is not None:
        np.testing.assert_array_equal(host(cu_blocks), ref_cub)


@pytest.mark.parametrize("wl_name,S,layout", CASES)
def test_indexer_score_tile(wl_name, S, layout):
    banner(f"score {wl_name} S={S} {layout}")
    wl, x = _inputs(wl_name, S, layout)
    d = _dev_inputs(wl, x)
    # the oracle's compressed keys feed both sides (FP32 copy for the GPU)
    kc_h, ref_cub = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, x["cu_seqlens"], x["row_lens"])
    kc = to_dev(kc_h.astype(np.float32))
    cu_blocks = to_dev(ref_cub)
    scale = 1.0 / math.sqrt(wl.D_idx)
    nb = S // wl.c
    # full tile plus an unaligned sub-tile
    for (q0, q1, j0, j1) in [(0, S, 0, nb), (S // 3 + 1, S - 7, nb // 5 + 3, nb - 2)]:
        out = irb.indexer_score_tile(d["qI"], d["w"], kc, wl.c, q0, q1, j0, j1, scale, cu_blocks, d["cu"], d["rl"])
        got = host(out)
        ref = oracle.indexer_scores(x["qI"], x["w"], kc_h, wl.c, scale, x["cu_seqlens"], x["row_lens"], q0, q1)[:, :, j0:j1]
        assert np.array_equal(np.isneginf(got), np.isneginf(ref))
        M = _score_bound(x["qI"][:, q0:q1], x["w"][:, q0:q1], kc_h[:, j0:j1], scale)
        fin = np.isfinite(ref)
        err = np.abs(got[fin] - ref[fin])
        # the FP32 scoring bound (well inside the stated 1e-3 relative)
        assert np.all(err <= SCORE_ERR * M[fin] + 1e-30), f"max rel-to-M {np.max(err / np.maximum(M[fin], 1e-30)):.2e}"


def _quantised_scores(rng, B, S, nb, ties):
    s = rng.standard_normal((B, S, nb))
    if ties:
        s = np.round(s * 2) / 2          # many exact ties, including 0.0
        s[rng.random(s.shape) < 0.1] = -0.0
    return s.astype(np.float32)


@pytest.mark.parametrize("layout,topk,c,S,ties", [
    ("single", 16, 4, 512, True), ("single", 512, 4, 8192, False), ("rows", 7, 2, 300, True),
    ("packed", 32, 4, 4096, True), ("single", 256, 8, 4096, True)])
def test_select_bit_exact_on_fixed_scores(layout, topk, c, S, ties):
    banner(f"select {layout} topk={topk} c={c} S={S} ties={ties}")
    rng = np.random.default_rng(topk + S)
    cu, rl, B = _layout_case(layout, S)
    nb = S // c
    scores = _quantised_scores(rng, B, S, nb, ties)
    sel, cnt = irb.select_topk_regions(to_dev(scores), c, topk, S, cu_blocks=_cu_blocks_dev(cu, c),
                                       cu_seqlens=to_dev(cu), row_lens=to_dev(rl))
    rsel, rcnt = oracle.select_topk(scores.astype(np.float64), c, topk, cu, rl)
    np.testing.assert_array_equal(host(cnt), rcnt)
    np.testing.assert_array_equal(host(sel), rsel)


def _cu_blocks_dev(cu, c):
    if cu is None:
        return None
    lens = np.diff(cu) // c
    return to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))


@pytest.mark.parametrize("wl_name,S,layout", [("tiny", 512, "single"), ("s8192", 2048, "single"),
                                              ("varlen", 4096, "packed"), ("long", 4096, "single"),
                                              ("s8192", 1500, "rows")])
def test_route_pipeline_matches_oracle(wl_name, S, layout):
    """compress -> fused score/select -> expand; every row bit-exact except near-tie rows, which
    must still hold a correct top-k under FP32 scoring and the expansion of the GPU's own selection."""
    banner(f"pipeline {wl_name} S={S} {layout}")
    wl, x = _inputs(wl_name, S, layout)
    d = _dev_inputs(wl, x)
    topk = min(wl.topk, max(4, S // wl.c // 4))     # keep selection sparse at reduced S
    r = irb.route(d["kI"], d["qI"], d["w"], d["gamma"], d["freqs"], wl.c, topk, wl.window, cu_seqlens=d["cu"],
                  row_lens=d["rl"])
    ref = oracle.route_pipeline(x["kI"], x["qI"], x["w"], x["gamma"], x["freqs"], wl.c, topk, wl.window,
                                cu_seqlens=x["cu_seqlens"], row_lens=x["row_lens"])
    ties = oracle.near_tie_rows(ref["scores"], wl.c, topk, x["cu_seqlens"], x["row_lens"])
    got = {k: host(r[k])[None] for k in ("sel", "cnt", "routes", "lens")}
    want = {k: ref[k][None] for k in ("sel", "cnt", "routes", "lens")}
    want["ties"] = ties[None]
    kc, _ = oracle.compress_keys(x["kI"], x["gamma"], 1e-5, x["freqs"], wl.c, x["cu_seqlens"], x["row_lens"])
    check_selection(wl, x, topk, got, want, kc, grouped=False)


@pytest.mark.parametrize("c,topk,window,layout,S", [(4, 16, 0, "single", 512), (4, 512, 128, "single", 8192),
                                                   (4, 8, 5, "packed", 3000), (8, 256, 512, "single", 8192),
                                                   (3, 5, 7, "rows", 400), (1, 6, 0, "rows", 300),
                                                   (3, 20, 8, "packed", 3000), (5, 40, 0, "single", 2048),
                                                   (16, 300, 64, "single", 8192)])
def test_expand_bit_exact_on_fixed_selection(c, topk, window, layout, S):
    banner(f"expand c={c} topk={topk} W={window} {layout} S={S}")
    rng = np.random.default_rng(S + c)
    cu, rl, B = _layout_case(layout, S)
    docs = oracle.documents(B, S, cu, rl)
    valid, start, base, nb = oracle.token_info(docs, S, c)
    sel = np.full((B, S, topk), -1, dtype=np.int32)
    cnt = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        for t in range(S):
            if valid[b, t] and nb[b, t]:
                k = min(topk, int(nb[b, t]))
                sel[b, t, :k] = np.sort(rng.choice(int(nb[b, t]), k, replace=False)) + base[b, t]
                cnt[b, t] = k
    routes, lens = irb.expand_and_compact_routes(to_dev(sel), to_dev(cnt), c, window, topk,
                                                 cu_blocks=_cu_blocks_dev(cu, c), cu_seqlens=to_dev(cu),
                                                 row_lens=to_dev(rl))
    rr, rl_ = oracle.expand_routes(sel, cnt, c, window, topk, cu, rl)
    np.testing.assert_array_equal(host(lens), rl_)
    np.testing.assert_array_equal(host(routes), rr)


@pytest.mark.parametrize("rows,width,key_count", [(300, 67, 300), (64, 2048, 5000), (17, 1, 3), (40, 1000, 10),
                                                  (50, 500, 1000000), (30, 3000, 70000)])
def test_compact_bit_exact(rows, width, key_count):
    banner(f"compact rows={rows} width={width} keys={key_count}")
    rng = np.random.default_rng(rows * width)
    ids = rng.integers(-3, key_count + 3, size=(rows, width)).astype(np.int32)
    out, lens, bad = irb.compact_routes(to_dev(ids), key_count)
    ro, rl, rbad = oracle.compact_routes(ids, key_count)
    np.testing.assert_array_equal(host(out), ro)
    np.testing.assert_array_equal(host(lens), rl)
    assert int(host(bad)[0]) == rbad
    # in place
    t = to_dev(ids)
    irb.compact_routes(t, key_count, out=t)
    np.testing.assert_array_equal(host(t), ro)


def test_compact_bitmap_capacity_edge():
    """Rows whose valid IDs span exactly the LDS bitmap's capacity (65536 values)
    and one more, with duplicates, invalid IDs and an all-invalid row."""
    banner("compact bitmap capacity edge")
    rng = np.random.default_rng(11)
    width, key_count = 700, 200000
    ids = rng.integers(1000, 1000 + 65536, size=(6, width)).astype(np.int32)
    ids[0, :2] = [1000, 1000 + 65535]          # span 65536 values
    ids[1, :2] = [1000, 1000 + 65536]          # span 65537 values
    ids[2, 1::3] = ids[2, ::3][: ids[2, 1::3].size]  # duplicates
    ids[3, ::2] = -1
    ids[4, 5] = key_count + 7                  # out of range, dropped and counted
    ids[5, :] = -5                             # nothing valid
    out, lens, bad = irb.compact_routes(to_dev(ids), key_count)
    ro, rl, rbad = oracle.compact_routes(ids, key_count)
    np.testing.assert_array_equal(host(out), ro)
    np.testing.assert_array_equal(host(lens), rl)
    assert int(host(bad)[0]) == rbad == 1


def test_compact_latent_indices():
    wl = synth.WORKLOADS["latent"]
    x = synth.make_inputs(wl, parts=("idx",), S=1024)
    banner("compact latent T=1024")
    out, lens, bad = irb.compact_routes(to_dev(x["idx"]), 1024)
    ro, rl, rbad = oracle.compact_routes(x["idx"], 1024)
    np.testing.assert_array_equal(host(out), ro)
    np.testing.assert_array_equal(host(lens), rl)
    assert rbad == 0 and int(host(bad)[0]) == 0


@pytest.mark.parametrize("bq,bk,reverse,width", [(1, 16, True, 40), (16, 64, False, 40), (16, 64, True, 40),
                                                 (3, 5, False, 40), (3, 5, True, 40), (128, 16, True, 40),
                                                 (1, 1, False, 40), (1, 16, True, 37), (3, 5, False, 301),
                                                 (1, 16, True, 600), (16, 64, False, 600)])
def test_block_lists_bit_exact(bq, bk, reverse, width):
    """Route widths that are a multiple of 4 take the 16-byte-load path, others
    the per-entry path; widths above 256 span several loads per lane."""
    banner(f"lists bq={bq} bk={bk} reverse={reverse} width={width}")
    rng = np.random.default_rng(bq * 100 + bk + width)
    B, S = 2, 700
    ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.2)
    routes, lens, _ = oracle.compact_routes(ids, S)
    counts, indices = irb.build_block_lists(to_dev(routes), to_dev(lens), S, bq, bk, reverse)
    rc, ri = oracle.block_lists(routes, lens, S, bq, bk, reverse)
    np.testing.assert_array_equal(host(counts), rc)
    np.testing.assert_array_equal(host(indices), ri)


@pytest.mark.parametrize("B,S_q,S_k,bq,width", [(2, 65560, 1000, 1, 24), (1, 131100, 1000, 2, 13)])
def test_reverse_lists_banded_bit_exact(B, S_q, S_k, bq, width):
    """Reverse lists with enough query tiles (over 65504) that the LDS band
    of the mark pass holds several words per key-tile row, the last band
    partial; key IDs past S_k are ignored; a 16-byte-load and a per-entry
    route width."""
    banner(f"banded reverse lists B={B} S_q={S_q} S_k={S_k} bq={bq} width={width}")
    rng = np.random.default_rng(S_q + width)
    ids = rng.integers(-1, S_k + 5, size=(B, S_q, width)).astype(np.int32)
    routes, lens, _ = oracle.compact_routes(ids, S_k)
    counts, indices = irb.build_block_lists(to_dev(routes), to_dev(lens), S_k, bq, 16, True)
    rc, ri = oracle.block_lists(routes, lens, S_k, bq, 16, True)
    np.testing.assert_array_equal(host(counts), rc)
    np.testing.assert_array_equal(host(indices), ri)


@pytest.mark.parametrize("ties", [False, True])
def test_select_rows_longer_than_lds(ties):
    """Rows with more visible blocks than the select kernel keeps in LDS (40000 > 32768)."""
    S, c, topk, rows = 160000, 4, 300, 16
    banner(f"select global-memory rows S={S} ties={ties}")
    rng = np.random.default_rng(7 + ties)
    q0 = S - rows
    scores = _quantised_scores(rng, 1, rows, S // c, ties)
    sel, cnt = irb.select_topk_regions(to_dev(scores), c, topk, S, q0=q0)
    rsel, rcnt = oracle.select_topk(scores.astype(np.float64), c, topk, q0=q0, S=S)
    np.testing.assert_array_equal(host(cnt)[:, q0:], rcnt)
    np.testing.assert_array_equal(host(sel)[:, q0:], rsel)


@pytest.mark.gpu
@pytest.mark.parametrize("S,c,topk", [(16384, 4, 512), (32768, 4, 256), (131072, 8, 256), (65536, 4, 300),
                                    (8192, 4, 100), (2048, 4, 64), (4096, 4, 1000)])
@pytest.mark.parametrize("ties", [False, True])
def test_select_long_rows(S, c, topk, ties):
    """Rows of 512 to 16384 visible blocks (every one-wave-per-row and
    register-resident width of the select kernels), with the last rows made
    constant, two-valued and of one repeated value above a sea of ties."""
    rows = 12
    banner(f"select long rows S={S} c={c} topk={topk} ties={ties}")
    rng = np.random.default_rng(S + topk + ties)
    q0 = S - rows
    nb = S // c
    scores = _quantised_scores(rng, 1, rows, nb, ties)
    scores[0, -1, :] = 0.25                                   # constant row: lowest IDs win
    scores[0, -2, :] = np.where(rng.random(nb) < 0.5, 1.0, -1.0).astype(np.float32)
    scores[0, -3, :] = -0.0
    scores[0, -3, rng.choice(nb, topk // 2, replace=False)] = 3.0
    sel, cnt = irb.select_topk_regions(to_dev(scores), c, topk, S, q0=q0)
    rsel, rcnt = oracle.select_topk(scores.astype(np.float64), c, topk, q0=q0, S=S)
    np.testing.assert_array_equal(host(cnt)[:, q0:], rcnt)
    np.testing.assert_array_equal(host(sel)[:, q0:], rsel)


@pytest.mark.parametrize("rows,slots,regions,sort", [(300, 67, 70, True), (64, 512, 2048, True), (17, 1, 1, False),
                                                     (40, 1000, 33, False), (9, 300, 131072, True), (5, 64, 4097, False),
                                                     (3, 4100, 5000, False), (4, 4100, 5000, True)])
def test_pack_region_bitmap_bit_exact(rows, slots, regions, sort):
    """Sorted and unsorted rows with repeats, -1 and at-or-above-regions padding;
    word counts from 1 to 4096 (the LDS limit)."""
    banner(f"bitmap rows={rows} slots={slots} regions={regions} sort={sort}")
    rng = np.random.default_rng(rows + slots + regions)
    ids = rng.integers(-2, regions + 3, size=(rows, slots)).astype(np.int32)
    if sort:
        ids.sort(axis=-1)
    got = irb.pack_region_bitmap(to_dev(ids), regions)
    np.testing.assert_array_equal(host(got), oracle.pack_region_bitmap(ids, regions))


def test_pack_region_bitmap_of_selected_blocks():
    """The S=8192 selection layout ([1, 8192, 512] ascending block ids, -1 padded) over 2048 regions."""
    wl = synth.WORKLOADS["s8192"]
    banner("bitmap of s8192-shaped selections")
    rng = np.random.default_rng(77)
    S, topk, nb = 8192, wl.topk, 8192 // wl.c
    sel = np.full((1, S, topk), -1, dtype=np.int32)
    for t in range(0, S, 97):
        n = (t + 1) // wl.c
        k = min(topk, n)
        sel[0, t, :k] = np.sort(rng.choice(n, k, replace=False)) if k else []
    got = irb.pack_region_bitmap(to_dev(sel), nb)
    np.testing.assert_array_equal(host(got), oracle.pack_region_bitmap(sel, nb))


def _split_check(routes, lens, S, bq, bk, reverse):
    r_d, l_d = to_dev(routes), to_dev(lens)
    counts, indices = irb.build_block_lists(r_d, l_d, S, bq, bk, reverse)
    rc, ri = oracle.block_lists(routes.reshape(-1, *routes.shape[-2:]), lens.reshape(-1, lens.shape[-1]), S, bq, bk,
                                reverse)
    np.testing.assert_array_equal(host(counts).reshape(rc.shape), rc)
    got = [host(x) for x in irb.split_full_blocks(r_d, l_d, S, bq, bk, reverse, counts, indices)]
    want = oracle.split_full_blocks(routes.reshape(-1, *routes.shape[-2:]), lens.reshape(-1, lens.shape[-1]), S, bq,
                                    bk, rc, ri, reverse)
    fc, fi, pc, pi = (g.reshape(w.shape) for g, w in zip(got, want))
    np.testing.assert_array_equal(fc, want[0], err_msg="full_counts")
    np.testing.assert_array_equal(pc, want[2], err_msg="part_counts")
    # entries past each count are not written: compare the listed prefixes
    valid_f = np.arange(fi.shape[-1]) < want[0][..., None]
    valid_p = np.arange(pi.shape[-1]) < want[2][..., None]
    np.testing.assert_array_equal(fi[valid_f], want[1][valid_f], err_msg="full_indices")
    np.testing.assert_array_equal(pi[valid_p], want[3][valid_p], err_msg="part_indices")
    if bq == 1:
        # one-query tiles: the coverage-bit path (above) and the route-search path agree
        other = [host(x) for x in irb.split_full_blocks(r_d, l_d, S, bq, bk, reverse, counts, indices,
                                                         use_workspace=False)]
        np.testing.assert_array_equal(other[0], got[0])
        np.testing.assert_array_equal(other[2], got[2])
        o1, o3 = other[1].reshape(fi.shape), other[3].reshape(pi.shape)
        np.testing.assert_array_equal(o1[valid_f], want[1][valid_f])
        np.testing.assert_array_equal(o3[valid_p], want[3][valid_p])
    print(f"  {int(want[0].sum())} full / {int(want[2].sum())} partial blocks")
    return int(want[0].sum())


@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 128), (16, 16), (1, 16), (5, 3)])
def test_split_full_blocks_pipeline_routes(bq, bk):
    """S=8192 recipe at S=2048 (all-selected prefix, then top-k blocks + 128-token
    window): full blocks in the prefix and along the window."""
    banner(f"split full blocks s8192 recipe S=2048 bq={bq} bk={bk}")
    wl = synth.WORKLOADS["s8192"]
    x = synth.make_inputs(wl, parts=("route",), S=2048)
    r = oracle.route_pipeline(x["kI"], x["qI"], x["w"], x["gamma"], x["freqs"], wl.c, 128, wl.window)
    nfull = 0
    for reverse in (False, True):
        nfull += _split_check(r["routes"], r["lens"], 2048, bq, bk, reverse)
    assert nfull > 0


@pytest.mark.parametrize("width,bq,bk", [(40, 3, 5), (300, 16, 16), (37, 1, 16), (64, 8, 1)])
def test_split_full_blocks_random_routes(width, bq, bk):
    """B=2 random causal routes with a dense causal prefix in row 0, an empty row and a ragged tail."""
    banner(f"split full blocks random width={width} bq={bq} bk={bk}")
    rng = np.random.default_rng(width + bq)
    B, S = 2, 333
    ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.2)
    routes, lens, _ = oracle.compact_routes(ids, S)
    for t in range(min(width, S)):
        routes[0, t] = -1
        routes[0, t, :t + 1] = np.arange(t + 1)
        lens[0, t] = t + 1
    routes[1, 7] = -1
    lens[1, 7] = 0
    for reverse in (False, True):
        _split_check(routes, lens, S, bq, bk, reverse)


def test_split_full_blocks_grouped_routes():
    """Per-KV-group routes [R, B, S, L] split as R * B route rows."""
    banner("split full blocks grouped routes")
    rng = np.random.default_rng(5)
    R, S, width = 4, 256, 128
    rs, ls = [], []
    for g in range(R):
        ids = synth.random_routes(rng, 1, S, width, causal=True, frac_invalid=0.1)
        r, n, _ = oracle.compact_routes(ids, S)
        for t in range(16 * g, min(S, 16 * g + 64)):
            r[0, t] = -1
            r[0, t, :t + 1] = np.arange(t + 1)
            n[0, t] = t + 1
        rs.append(r)
        ls.append(n)
    for reverse in (False, True):
        _split_check(np.stack(rs), np.stack(ls), S, 8, 8, reverse)
