"""Pins of the CSA-variant oracle functions (CSA page: gather_region_payload,
_summarize_region_payload, indexer_score_tile's E4M3-rounded inputs,
RegionSelection.region_ids with RegionMetadata.current)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden


# ---------------------------------------------------------------- roundings
def _e4m3_values():
    """Every finite E4M3 value from the format's definition (sign, 4-bit
    exponent with bias 7, 3-bit mantissa; exponent field 0 = subnormals;
    S.1111.111 is NaN)."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
            vals += [v, -v]
    return np.unique(np.array(vals))


def test_e4m3_grid_is_the_format():
    vals = _e4m3_values()
    assert vals.max() == 448.0 and np.min(vals[vals > 0]) == 2.0 ** -9
    np.testing.assert_array_equal(oracle.round_to_e4m3(vals), vals)      # every code is a fixed point


def test_e4m3_matches_torch_float8_cast():
    """torch's float8_e4m3fn conversion (a library routine): random magnitudes
    over the whole range, every midpoint between neighbouring codes (ties go
    to the even code), the overflow boundary and specials."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-14, 7, 200000))
    pos = _e4m3_values()[_e4m3_values() >= 0]
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([x, mids, -mids, [463.99, 464.0, 464.01, 479.0, 480.0, 1e6, np.inf, -np.inf, np.nan, 0.0, -0.0]])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.round_to_e4m3(x32.astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x32[~same][:10]
    assert np.signbit(oracle.round_to_e4m3(np.array([-0.0])))[0]


def test_e4m3_hand_values():
    cases = {1.0625: 1.0, 1.1875: 1.25, 17.0: 16.0, 19.0: 20.0, 0.0009765625: 0.0, 0.0029296875: 0.00390625,
             464.0: 448.0, -300.0: -288.0}
    for x, y in cases.items():
        assert oracle.round_to_e4m3(np.array([x]))[0] == y, x
    assert np.isnan(oracle.round_to_e4m3(np.array([465.0]))[0])


def test_bf16_matches_torch():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-40, 40, 100000))).astype(np.float32)
    # halfway cases: the low 16 bits exactly 0x8000
    h = (rng.integers(0, 2 ** 15, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, h[np.isfinite(h)]])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)), want)


# ---------------------------------------------------------------- gather
def test_gather_region_payload_fixture():
    g = load_golden("region_payload_tiny.json")
    keys = np.array(g["keys"], dtype=np.float32)
    logits = np.array(g["logits"], dtype=np.float32)
    src = np.array(g["sources"], dtype=np.int32)
    valid = np.array(g["valid"], dtype=bool)
    pk, pz = oracle.gather_region_payload(keys, logits, src, valid)
    np.testing.assert_array_equal(pk, np.array(g["packed_keys"], dtype=np.float32))
    np.testing.assert_array_equal(pz, np.array(g["packed_logits"], dtype=np.float32))


def test_gather_region_payload_invariants():
    rng = np.random.default_rng(9)
    B, T, D, R, rs = 2, 37, 8, 11, 4
    keys = rng.standard_normal((B, T, D)).astype(np.float32)
    logits = rng.standard_normal((B, T, D)).astype(np.float32)
    src = rng.integers(-1, T, (B, R, rs)).astype(np.int32)
    valid = (src >= 0) & (rng.random((B, R, rs)) < 0.8)
    pk, pz = oracle.gather_region_payload(keys, logits, src, valid)
    for b, r, s in itertools.product(range(B), range(R), range(rs)):
        if valid[b, r, s]:
            assert np.array_equal(pk[b, r, s], keys[b, src[b, r, s]])
            assert np.array_equal(pz[b, r, s], logits[b, src[b, r, s]])
        else:
            assert not pk[b, r, s].any() and not pz[b, r, s].any()


# ---------------------------------------------------------------- summaries
def _one_region(k_rows, z_rows, valid=None):
    k = np.array(k_rows, dtype=np.float32)[None, None]
    z = np.array(z_rows, dtype=np.float32)[None, None]
    v = np.ones(k.shape[:3], dtype=bool) if valid is None else np.array(valid, dtype=bool)[None, None]
    return oracle.summarize_region_payload(k, z, v)[0, 0]


def test_summary_equal_logits_is_the_mean():
    k = [[1.0, -2.0, 0.5, 3.0], [3.0, 2.0, 0.25, -1.0], [5.0, 0.0, 0.75, 1.0], [7.0, 4.0, 2.5, 1.0]]
    z = [[0.3] * 4] * 4
    np.testing.assert_array_equal(_one_region(k, z), oracle.round_to_e4m3(np.mean(np.array(k), axis=0)))


def test_summary_single_valid_slot_and_dominant_logit():
    k = [[1.3, -0.7], [9.0, 9.0], [2.2, 0.01]]
    # only slot 0 valid: its key, rounded twice
    np.testing.assert_array_equal(_one_region(k, [[0, 0]] * 3, [True, False, False]),
                                  oracle.round_to_e4m3(oracle.round_to_bf16(np.float32([1.3, -0.7]))))
    # slot 2 dominates dim 0 and slot 0 dominates dim 1: exp(-100) vanishes in float32
    got = _one_region(k, [[0.0, 100.0], [0.0, 0.0], [100.0, 0.0]])
    np.testing.assert_array_equal(got, oracle.round_to_e4m3(oracle.round_to_bf16(np.float32([2.2, -0.7]))))


def test_summary_rounds_to_bf16_before_e4m3():
    """1.0655 lies above the E4M3 midpoint 1.0625, so rounding it straight to
    E4M3 gives 1.125; the BF16 rounding first lands on the midpoint itself,
    which then goes to the even code 1.0."""
    assert oracle.round_to_e4m3(np.array([1.0655]))[0] == 1.125
    assert _one_region([[1.0655]], [[0.0]])[0] == 1.0


def test_summary_empty_region_is_zero():
    assert not _one_region([[1.0, 2.0]], [[0.0, 0.0]], [False]).any()


# ---------------------------------------------------------------- selection with the current region
def _scores(rng, S, nb, ties):
    s = rng.standard_normal((1, S, nb))
    return np.round(s * 2) / 2 if ties else s


@pytest.mark.parametrize("layout", ["single", "packed"])
def test_select_regions_csa_brute_force(layout):
    rng = np.random.default_rng(10)
    c, topk = 3, 2
    if layout == "single":
        S, cu = 20, None
    else:
        S, cu = 24, np.array([0, 7, 15, 22], dtype=np.int32)      # lengths 7, 8, 7 and 2 padding tokens
    docs = oracle.documents(1, S, cu, None)
    valid, start, base, nb = oracle.token_info(docs, S, c)
    NB = int(sum((e - a) // c for a, e in docs[0]))
    rbases, totals = oracle.region_bases(docs, c)
    R = totals[0]
    assert R == sum(-(-(e - a) // c) for a, e in docs[0])          # incomplete last regions count
    for trial in range(20):
        sc = _scores(rng, S, NB, ties=trial % 2 == 0)
        ids, cnt = oracle.select_regions_csa(sc, c, topk, cu)
        for t in range(S):
            row, n = ids[0, t], int(cnt[0, t])
            if not valid[0, t]:
                assert n == 0 and (row == R).all()
                continue
            d = [a for a, e in docs[0]].index(int(start[0, t]))
            pos = t - int(start[0, t])
            h = pos // c
            assert n == min(topk, h) + 1
            assert (row[n:] == R).all() and np.all(np.diff(row[:n]) > 0)
            assert row[n - 1] == rbases[0][d] + h                      # the current region, last
            chosen = row[:n - 1] - rbases[0][d]
            assert np.all((chosen >= 0) & (chosen < h))
            # brute force: the chosen set maximises the score sum, ties to the lower ids
            vis = sc[0, t, int(base[0, t]):int(base[0, t]) + h]
            best = max(itertools.combinations(range(h), len(chosen)),
                       key=lambda cmb: (sorted(vis[list(cmb)].tolist(), reverse=True), [-i for i in cmb]))
            assert sorted(vis[chosen].tolist(), reverse=True) == sorted(vis[list(best)].tolist(), reverse=True)


def test_select_regions_csa_matches_select_topk_away_from_block_ends():
    """Where the query's own group is incomplete ((pos + 1) % c != 0) the
    historical regions are exactly the visible complete blocks, so the
    selection equals select_topk's (single document: same numbering)."""
    rng = np.random.default_rng(11)
    S, c, topk = 64, 4, 5
    sc = rng.standard_normal((1, S, S // c))
    ids, cnt = oracle.select_regions_csa(sc, c, topk)
    sel, scnt = oracle.select_topk(sc, c, topk)
    for t in range(S):
        if (t + 1) % c == 0:
            continue
        k = int(scnt[0, t])
        np.testing.assert_array_equal(ids[0, t, :k], sel[0, t, :k])
        assert ids[0, t, k] == t // c and cnt[0, t] == k + 1
