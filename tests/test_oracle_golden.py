"""Oracle against hand-derived fixtures (tests/golden/*.json, each with its derivation)."""
import math

import numpy as np
import pytest

import oracle
from conftest import as_float, load_golden


def test_compress_full_and_half_rope():
    g = load_golden("compress_tiny.json")
    kI = np.array(g["kI"], dtype=np.float64)[None]
    for table, key in (("freqs_full", "expected_full"), ("freqs_half", "expected_half")):
        freqs = np.array(g[table], dtype=np.float64)[None]
        kc, cu_blocks = oracle.compress_keys(kI, g["gamma"], g["eps"], freqs, g["c"])
        assert cu_blocks is None
        np.testing.assert_allclose(kc[0], np.array(g[key]), rtol=0, atol=1e-12)


def test_scores_by_hand():
    g = load_golden("scores_tiny.json")
    kc = np.array(g["kc"], dtype=np.float64)[None]
    qI = np.array(g["qI"], dtype=np.float64)[None]
    w = np.array(g["w"], dtype=np.float64)[None]
    s = oracle.indexer_scores(qI, w, kc, g["c"], scale=g["scale"])
    exp = np.array(as_float(g["expected"]))
    assert np.array_equal(np.isinf(s[0]), np.isinf(exp))
    np.testing.assert_allclose(s[0][np.isfinite(exp)], exp[np.isfinite(exp)], rtol=0, atol=1e-12)


def test_select_by_hand():
    g = load_golden("select_tiny.json")
    for case in g["cases"]:
        row = np.array(as_float(case["scores"]), dtype=np.float64)
        n, k = len(row), case["topk"]
        # one query at document position n*1 - 1 with c=1 sees all n blocks
        S = n
        scores = np.full((1, S, n), -np.inf)
        scores[0, S - 1] = row
        sel, cnt = oracle.select_topk(scores, 1, k)
        assert sel[0, S - 1].tolist() == case["expected"], case
        assert cnt[0, S - 1] == min(k, n)


def test_routes_by_hand():
    g = load_golden("routes_tiny.json")
    S, c, topk, W = g["S"], g["c"], g["topk"], g["window"]
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    sel = np.full((1, S, topk), -1, dtype=np.int32)
    cnt = np.zeros((1, S), dtype=np.int32)
    for t, ids in g["rows"].items():
        sel[0, int(t), :len(ids)] = ids
        cnt[0, int(t)] = len(ids)
    routes, lens = oracle.expand_routes(sel, cnt, c, W, topk, cu_seqlens=cu)
    assert routes.shape[-1] == 11 == oracle.route_width(topk, c, W)
    for t, exp in g["expected"].items():
        t = int(t)
        assert lens[0, t] == len(exp)
        assert routes[0, t].tolist() == exp + [-1] * (11 - len(exp))


def test_compact_by_hand():
    g = load_golden("compact_tiny.json")
    out, lens, bad = oracle.compact_routes(np.array(g["ids"]), g["key_count"])
    assert out.tolist() == g["expected"]
    assert lens.tolist() == g["lens"]
    assert bad == g["out_of_range"]


def test_block_lists_by_hand():
    g = load_golden("block_lists_tiny.json")
    routes = np.array(g["routes"], dtype=np.int32)[None]
    lens = np.array(g["lens"], dtype=np.int32)[None]
    c, i = oracle.block_lists(routes, lens, g["S_k"], g["block_q"], g["block_k"], reverse=False)
    assert c[0].tolist() == g["fwd_counts"] and i[0].tolist() == g["fwd_indices"]
    c, i = oracle.block_lists(routes, lens, g["S_k"], g["block_q"], g["block_k"], reverse=True)
    assert c[0].tolist() == g["rev_counts"] and i[0].tolist() == g["rev_indices"]


def test_attention_by_hand():
    g = load_golden("attention_tiny.json")
    A = g["A"]
    q = np.array(A["q"], dtype=np.float64)[None]
    k = np.array(A["k"], dtype=np.float64)[None]
    v = np.array(A["v"], dtype=np.float64)[None]
    routes = np.array([[A["route"]]], dtype=np.int32)
    o, lse = oracle.attention_fwd(q, k, v, routes, scale=A["scale"])
    np.testing.assert_allclose(o[0, 0], np.array(A["expected_o"]), atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], np.array(A["expected_lse"]), atol=1e-12)
    assert math.isclose(A["expected_lse"][0], math.log(4.0))
    Bc = g["B"]
    q = np.array(Bc["q"], dtype=np.float64)[None, None]
    k = np.array(Bc["k"], dtype=np.float64)[None]
    v = np.array(Bc["v"], dtype=np.float64)[None]
    routes = np.array([[Bc["route"]]], dtype=np.int32)
    o, _ = oracle.attention_fwd(q, k, v, routes)
    np.testing.assert_allclose(o[0, 0], np.array(Bc["expected_o"]), atol=1e-12)
