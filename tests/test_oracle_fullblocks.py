"""Pins of the oracle's full/partial block split: a hand-written case, the closed
form of complete causal rectangles for all-selected routes, the FA4 page's
all-selected-prefix rule, and partition / forward-reverse invariants."""
import numpy as np
import pytest

import oracle
import synth


def _routes_from_sets(sets, L):
    S = len(sets)
    r = np.full((1, S, L), -1, dtype=np.int32)
    n = np.zeros((1, S), dtype=np.int32)
    for t, s in enumerate(sets):
        ids = sorted(s)
        r[0, t, :len(ids)] = ids
        n[0, t] = len(ids)
    return r, n


def _split(routes, lens, S_k, bq, bk, reverse):
    c, i = oracle.block_lists(routes, lens, S_k, bq, bk, reverse=reverse)
    return (c, i) + oracle.split_full_blocks(routes, lens, S_k, bq, bk, c, i, reverse=reverse)


def _pairs(c, i, reverse):
    out = set()
    for b in range(c.shape[0]):
        for r in range(c.shape[1]):
            for e in range(c[b, r]):
                out.add((b, int(i[b, r, e]), r) if reverse else (b, r, int(i[b, r, e])))
    return out


def test_hand_written_case():
    # queries 0..3, tiles of 2 queries and 2 keys
    routes, lens = _routes_from_sets([{0}, {0, 1}, {0, 1, 2}, {0, 1, 2, 3}], 4)
    c, i, fc, fi, pc, pi = _split(routes, lens, 4, 2, 2, False)
    # q-tile 0: key tile 0 misses (0, 1); q-tile 1: key tile 0 complete, key tile 1 misses (2, 3)
    assert c.tolist() == [[1, 2]]
    assert fc.tolist() == [[0, 1]] and fi[0, 1, :1].tolist() == [0]
    assert pc.tolist() == [[1, 1]] and pi[0, 0, :1].tolist() == [0] and pi[0, 1, :1].tolist() == [1]
    c, i, fc, fi, pc, pi = _split(routes, lens, 4, 2, 2, True)
    # key tile 0: q-tile 0 partial, q-tile 1 full; key tile 1: q-tile 1 partial
    assert fc.tolist() == [[1, 0]] and fi[0, 0, :1].tolist() == [1]
    assert pc.tolist() == [[1, 1]] and pi[0, 0, :1].tolist() == [0] and pi[0, 1, :1].tolist() == [1]


@pytest.mark.parametrize("S,bq,bk", [(37, 5, 3), (64, 16, 16), (50, 1, 16), (40, 8, 1), (33, 4, 7)])
def test_all_selected_causal_routes_closed_form(S, bq, bk):
    """Every query routes to all keys up to itself: the full blocks are exactly the
    rectangles whose last key is at or below their first query."""
    routes, lens = _routes_from_sets([set(range(t + 1)) for t in range(S)], S)
    for reverse in (False, True):
        c, i, fc, fi, pc, pi = _split(routes, lens, S, bq, bk, reverse)
        got = _pairs(fc, fi, reverse)
        want = {(0, qi, kj) for (_, qi, kj) in _pairs(c, i, reverse)
                if min((kj + 1) * bk, S) - 1 <= qi * bq}
        assert got == want
        assert _pairs(pc, pi, reverse) == _pairs(c, i, reverse) - want


@pytest.mark.parametrize("p", [0, 20, 48])
def test_all_selected_prefix_rule(p):
    """FA4 page: with an all-selected query prefix of length p, the complete causal
    rectangles of query tiles inside the prefix are full; rows past it route sparsely."""
    rng = np.random.default_rng(200 + p)
    S, bq, bk = 64, 8, 4
    sets = []
    for t in range(S):
        if t < p:
            sets.append(set(range(t + 1)))
        else:
            keep = rng.random(t + 1) < 0.5
            keep[t] = True
            keep[0] = False                  # every sparse row misses key 0
            sets.append(set(np.nonzero(keep)[0].tolist()))
    routes, lens = _routes_from_sets(sets, S)
    c, i, fc, fi, pc, pi = _split(routes, lens, S, bq, bk, False)
    full = _pairs(fc, fi, False)
    for (_, qi, kj) in _pairs(c, i, False):
        in_prefix = min((qi + 1) * bq, S) <= p
        causal_complete = min((kj + 1) * bk, S) - 1 <= qi * bq
        if in_prefix and causal_complete:
            assert (0, qi, kj) in full
        if kj == 0 and min((qi + 1) * bq, S) > p:
            assert (0, qi, kj) not in full   # a sparse row of the tile misses key 0


def test_partition_and_forward_reverse_agree():
    rng = np.random.default_rng(7)
    B, S, width = 2, 45, 30
    ids = synth.random_routes(rng, B, S, width, causal=True, frac_invalid=0.2)
    routes, lens, _ = oracle.compact_routes(ids, S)
    # make some rows dense so that full blocks occur
    for t in range(0, 20):
        routes[0, t] = -1
        routes[0, t, :t + 1] = np.arange(t + 1)
        lens[0, t] = t + 1
    routes[1, 3] = -1
    lens[1, 3] = 0
    fwd = _split(routes, lens, S, 4, 3, False)
    rev = _split(routes, lens, S, 4, 3, True)
    for (c, i, fc, fi, pc, pi), reverse in ((fwd, False), (rev, True)):
        np.testing.assert_array_equal(fc + pc, c)
        for b in range(B):
            for r in range(c.shape[1]):
                merged = sorted(fi[b, r, :fc[b, r]].tolist() + pi[b, r, :pc[b, r]].tolist())
                assert merged == i[b, r, :c[b, r]].tolist()
                # order kept: each part ascending, -1 after the count
                assert list(fi[b, r, :fc[b, r]]) == sorted(fi[b, r, :fc[b, r]])
                assert np.all(fi[b, r, fc[b, r]:] == -1) and np.all(pi[b, r, pc[b, r]:] == -1)
    assert _pairs(fwd[2], fwd[3], False) == _pairs(rev[2], rev[3], True)
    assert len(_pairs(fwd[2], fwd[3], False)) > 0


def test_empty_routes_have_no_full_blocks():
    routes = np.full((1, 10, 4), -1, dtype=np.int32)
    lens = np.zeros((1, 10), dtype=np.int32)
    routes[0, 9, 0] = 3
    lens[0, 9] = 1
    c, i, fc, fi, pc, pi = _split(routes, lens, 10, 1, 1, False)
    # a 1x1 rectangle holding the routed pair is full; nothing else is listed
    assert c.sum() == 1 and fc.sum() == 1
    c, i, fc, fi, pc, pi = _split(routes, lens, 10, 2, 2, False)
    assert c.sum() == 1 and fc.sum() == 0 and pc.sum() == 1
