"""Pins of the oracle's scoring and top-k selection: brute force and invariants."""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _is_topk_set(row, chosen):
    """Definition: every chosen block beats every unchosen one (ties -> lower ID)."""
    others = [j for j in range(len(row)) if j not in chosen]
    for i in chosen:
        for j in others:
            if not (row[i] > row[j] or (row[i] == row[j] and i < j)):
                return False
    return True


def test_select_matches_subset_enumeration():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 6))
        vals = rng.integers(-2, 3, size=n).astype(np.float64)   # many exact ties
        vals[rng.random(n) < 0.2] = -0.0
        scores = np.full((1, n, n), -np.inf)
        scores[0, n - 1] = vals
        sel, cnt = oracle.select_topk(scores, 1, k)
        got = [int(x) for x in sel[0, n - 1] if x >= 0]
        keff = min(k, n)
        winners = [set(s) for s in itertools.combinations(range(n), keff) if _is_topk_set(vals, set(s))]
        assert len(winners) == 1
        assert got == sorted(winners[0])
        assert cnt[0, n - 1] == keff
        assert all(x == -1 for x in sel[0, n - 1, keff:])


def _pipeline_inputs(S=96, c=4, H=3, D=8, cu=None, row_lens=None, B=1, seed=3):
    rng = np.random.default_rng(seed)
    kI = rng.standard_normal((B, S, D))
    qI = rng.standard_normal((B, S, H, D))
    w = rng.standard_normal((B, S, H))
    freqs = synth.rope_table(synth.doc_positions(B, S, cu, row_lens), D).astype(np.float64)
    kc, cu_blocks = oracle.compress_keys(kI, np.ones(D), 1e-5, freqs, c, cu, row_lens)
    return kc, cu_blocks, qI, w


def test_score_visibility_and_document_confinement():
    cu = np.array([0, 10, 11, 50, 90], dtype=np.int32)
    c = 4
    kc, cu_blocks, qI, w = _pipeline_inputs(S=96, c=c, cu=cu)
    s = oracle.indexer_scores(qI, w, kc, c, cu_seqlens=cu)
    for t in range(96):
        fin = np.nonzero(np.isfinite(s[0, t]))[0]
        if t >= cu[-1]:
            assert len(fin) == 0
            continue
        d = int(np.searchsorted(cu, t, side="right") - 1)
        nb = (t - cu[d] + 1) // c
        assert fin.tolist() == list(range(cu_blocks[d], cu_blocks[d] + nb))


def test_score_homogeneity_sign_and_head_permutation():
    c = 2
    kc, _, qI, w = _pipeline_inputs(S=40, c=c)
    s = oracle.indexer_scores(qI, w, kc, c)
    fin = np.isfinite(s)
    s2 = oracle.indexer_scores(2.5 * qI, w, kc, c)          # relu is positively homogeneous
    np.testing.assert_allclose(s2[fin], 2.5 * s[fin], rtol=1e-12)
    s3 = oracle.indexer_scores(qI, -w, kc, c)               # signed weights flip the sign
    np.testing.assert_allclose(s3[fin], -s[fin], rtol=1e-12)
    perm = [2, 0, 1]
    s4 = oracle.indexer_scores(qI[:, :, perm], w[:, :, perm], kc, c)
    np.testing.assert_allclose(s4[fin], s[fin], rtol=1e-12)
    s5 = oracle.indexer_scores(qI, w, kc, c, scale=1.0)
    np.testing.assert_allclose(s5[fin] / np.sqrt(8.0), s[fin], rtol=1e-12)
    # a head whose weight is zero does not matter
    w0 = w.copy(); w0[:, :, 1] = 0
    q0 = qI.copy(); q0[:, :, 1] = 1e3
    s6 = oracle.indexer_scores(qI, w0, kc, c)
    s7 = oracle.indexer_scores(q0, w0, kc, c)
    np.testing.assert_array_equal(s6, s7)


def test_score_chunk_invariance():
    c = 4
    kc, _, qI, w = _pipeline_inputs(S=96, c=c)
    full = oracle.indexer_scores(qI, w, kc, c)
    parts = [oracle.indexer_scores(qI, w, kc, c, q0=a, q1=min(96, a + 17), row_chunk=5) for a in range(0, 96, 17)]
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), full)
    sel, cnt = oracle.select_topk(full, c, 5)
    sels = [oracle.select_topk(full[:, a:a + 17], c, 5, q0=a, S=96) for a in range(0, 96, 17)]
    np.testing.assert_array_equal(np.concatenate([x[0] for x in sels], axis=1), sel)


@pytest.mark.parametrize("layout", ["rows", "packed"])
def test_selection_invariants(layout):
    c, topk = 4, 3
    if layout == "packed":
        cu = np.array([0, 7, 40, 41, 88], dtype=np.int32); rl = None; B = 1
    else:
        cu = None; rl = np.array([96, 33]); B = 2
    kc, cu_blocks, qI, w = _pipeline_inputs(S=96, c=c, cu=cu, row_lens=rl, B=B)
    s = oracle.indexer_scores(qI, w, kc, c, cu_seqlens=cu, row_lens=rl)
    sel, cnt = oracle.select_topk(s, c, topk, cu_seqlens=cu, row_lens=rl)
    docs = oracle.documents(B, 96, cu, rl)
    valid, start, base, nb = oracle.token_info(docs, 96, c)
    for b in range(B):
        for t in range(96):
            row = sel[b, t]
            k = int(cnt[b, t])
            if not valid[b, t]:
                assert k == 0 and np.all(row == -1)
                continue
            assert k == min(topk, nb[b, t])
            ids = row[:k]
            assert np.all(np.diff(ids) > 0) and np.all(row[k:] == -1)
            assert np.all(ids >= base[b, t]) and np.all(ids < base[b, t] + nb[b, t])
            if nb[b, t] <= topk:
                assert ids.tolist() == list(range(base[b, t], base[b, t] + nb[b, t]))
            else:
                vis = s[b, t, base[b, t]:base[b, t] + nb[b, t]]
                chosen = set((ids - base[b, t]).tolist())
                assert _is_topk_set(vis, chosen)


def test_near_tie_detection():
    scores = np.full((1, 6, 6), -np.inf)
    scores[0, 5] = [1.0, 2.0, 2.00001, 0.5, 3.0, -1.0]
    scores[0, 4, :5] = [1.0, 2.0, 2.00001, 0.5, 3.0]
    # top-2 boundary: 2.00001 against 2.0 -> near tie in both rows
    ties = oracle.near_tie_rows(scores, 1, 2)
    assert ties[0, 4] and ties[0, 5]
    # top-3 boundary: 2.0 against 1.0 -> clear
    assert not oracle.near_tie_rows(scores, 1, 3)[0, 4:].any()
    # rows that see no more than topk blocks are never near ties
    assert not oracle.near_tie_rows(scores, 1, 6).any()
    # exact zero ties count as near ties
    z = np.full((1, 4, 4), -np.inf)
    z[0, 3] = [0.0, 0.0, -0.0, 1.0]
    assert oracle.near_tie_rows(z, 1, 2)[0, 3]
