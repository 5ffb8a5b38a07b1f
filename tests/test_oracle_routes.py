"""Pins of the oracle's route expansion, compaction and block lists: invariants and brute force."""
import numpy as np
import pytest

import oracle
import synth


def _random_selection(rng, docs, S, c, topk, B):
    """Any valid selection: k_eff distinct visible blocks per query, ascending."""
    valid, start, base, nb = oracle.token_info(docs, S, c)
    sel = np.full((B, S, topk), -1, dtype=np.int32)
    cnt = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        for t in range(S):
            if not valid[b, t] or nb[b, t] == 0:
                continue
            k = min(topk, int(nb[b, t]))
            ids = np.sort(rng.choice(int(nb[b, t]), size=k, replace=False)) + base[b, t]
            sel[b, t, :k] = ids
            cnt[b, t] = k
    return sel, cnt, valid, start, base, nb


@pytest.mark.parametrize("c,topk,window,layout", [
    (4, 3, 0, "packed"), (4, 3, 6, "packed"), (3, 2, 5, "rows"), (8, 2, 1, "rows"), (1, 4, 0, "rows"), (2, 5, 16, "packed")])
def test_route_invariants(c, topk, window, layout):
    rng = np.random.default_rng(21)
    S = 90
    if layout == "packed":
        cu = np.array([0, 5, 6, 47, 80], dtype=np.int32); rl = None; B = 1
    else:
        cu = None; rl = np.array([90, 41, 2]); B = 3
    docs = oracle.documents(B, S, cu, rl)
    sel, cnt, valid, start, base, nb = _random_selection(rng, docs, S, c, topk, B)
    routes, lens = oracle.expand_routes(sel, cnt, c, window, topk, cu, rl)
    L = oracle.route_width(topk, c, window)
    assert routes.shape == (B, S, L)
    for b in range(B):
        for t in range(S):
            n = int(lens[b, t])
            r = routes[b, t]
            if not valid[b, t]:
                assert n == 0 and np.all(r == -1)
                continue
            ids = r[:n]
            assert np.all(r[n:] == -1) and n <= L
            assert np.all(np.diff(ids) > 0)                       # ascending, unique
            assert ids[0] >= start[b, t] and ids[-1] <= t          # in-document and causal
            a = int(start[b, t])
            tail = set(range(a + int(nb[b, t]) * c, t + 1))
            win = set(range(max(a, t - window + 1), t + 1)) if window else set()
            blocks = {a + (int(j) - int(base[b, t])) * c + o for j in sel[b, t, :cnt[b, t]] for o in range(c)}
            assert tail <= set(ids.tolist()) and win <= set(ids.tolist())
            # size: c*k_eff + |tail u win| - overlap between blocks and the window
            assert n == c * int(cnt[b, t]) + len(tail | win) - len(blocks & (tail | win))
            # nothing outside blocks, tail and window
            assert set(ids.tolist()) == blocks | tail | win


def test_full_prefix_when_everything_is_selected():
    c, S = 4, 50
    cu = np.array([0, 13, 50], dtype=np.int32)
    docs = oracle.documents(1, S, cu, None)
    valid, start, base, nb = oracle.token_info(docs, S, c)
    topk = 100
    sel = np.full((1, S, topk), -1, dtype=np.int32)
    cnt = np.zeros((1, S), dtype=np.int32)
    for t in range(S):
        n = int(nb[0, t])
        sel[0, t, :n] = np.arange(n) + base[0, t]
        cnt[0, t] = n
    routes, lens = oracle.expand_routes(sel, cnt, c, 0, topk, cu)
    for t in range(S):
        assert routes[0, t, :lens[0, t]].tolist() == list(range(int(start[0, t]), t + 1))


def test_compaction_against_python_sets():
    rng = np.random.default_rng(22)
    ids = synth.random_routes(rng, 2, 40, 24, causal=True, frac_invalid=0.2)
    out, lens, bad = oracle.compact_routes(ids, 40)
    exp_bad = 0
    for b in range(2):
        for t in range(40):
            row = [int(x) for x in ids[b, t]]
            exp_bad += sum(1 for x in row if x >= 40)
            want = sorted({x for x in row if 0 <= x < 40})
            assert lens[b, t] == len(want)
            assert out[b, t].tolist() == want + [-1] * (24 - len(want))
    assert bad == exp_bad


@pytest.mark.parametrize("bq,bk", [(1, 1), (2, 4), (16, 64), (3, 5)])
def test_block_lists_brute_force_and_transpose(bq, bk):
    rng = np.random.default_rng(23)
    B, S = 2, 77
    routes = synth.random_routes(rng, B, S, 12, causal=True, frac_invalid=0.0)
    routes, lens, _ = oracle.compact_routes(routes, S)
    lens[1, 5:9] = 0
    routes[1, 5:9] = -1
    fc, fi = oracle.block_lists(routes, lens, S, bq, bk, reverse=False)
    rc, ri = oracle.block_lists(routes, lens, S, bq, bk, reverse=True)
    nqt, nkt = -(-S // bq), -(-S // bk)
    for b in range(B):
        pairs = set()
        for t in range(S):
            for k in routes[b, t, :lens[b, t]]:
                pairs.add((t // bq, int(k) // bk))
        for i in range(nqt):
            want = sorted(j for (a, j) in pairs if a == i)
            assert fc[b, i] == len(want) and fi[b, i, :len(want)].tolist() == want
            assert np.all(fi[b, i, len(want):] == -1)
        for j in range(nkt):
            want = sorted(i for (i, a) in pairs if a == j)
            assert rc[b, j] == len(want) and ri[b, j, :len(want)].tolist() == want
        # reverse lists are the transpose of forward lists
        assert sum(fc[b]) == sum(rc[b]) == len(pairs)


@pytest.mark.parametrize("bq,bk,reverse", [(1, 16, True), (4, 8, False), (3, 5, True), (16, 64, False)])
def test_block_lists_row_subset_matches_full(bq, bk, reverse):
    rng = np.random.default_rng(91)
    ids = synth.random_routes(rng, 2, 70, 23, causal=True, frac_invalid=0.3)
    routes, lens, _ = oracle.compact_routes(ids, 70)
    full_c, full_i = oracle.block_lists(routes, lens, 70, bq, bk, reverse)
    n_rows = full_c.shape[1]
    want = [(b, r) for b in range(2) for r in range(n_rows) if (b + r) % 3 != 1]
    part_c, part_i = oracle.block_lists(routes, lens, 70, bq, bk, reverse, rows=want)
    for b, r in want:
        assert part_c[b, r] == full_c[b, r]
        np.testing.assert_array_equal(part_i[b, r], full_i[b, r])
