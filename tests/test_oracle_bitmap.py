"""Pins of the oracle's region bitmap packer (CSA page, pack_region_bitmap)."""
import numpy as np
import pytest

import oracle


def test_hand_written_rows():
    """Row 0: regions 0, 1, 31, 32 and 69 (two words plus a third, 70 regions);
    row 1: only padding (70, a large id, -1); row 2: a repeated id."""
    ids = np.array([[0, 1, 31, 32, 69, 70], [70, 1000, -1, 70, 70, 70], [5, 5, 5, 70, 70, 70]], dtype=np.int32)
    got = oracle.pack_region_bitmap(ids, 70).view(np.uint32)
    want = np.array([[0x80000003, 0x00000001, 0x00000020], [0, 0, 0], [0x20, 0, 0]], dtype=np.uint32)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("regions,slots", [(1, 3), (31, 10), (32, 40), (33, 5), (200, 64), (1000, 300)])
def test_matches_set_membership_and_popcount(regions, slots):
    rng = np.random.default_rng(regions * 7 + slots)
    ids = rng.integers(-3, regions + 5, size=(2, 3, 9, slots)).astype(np.int32)
    ids.sort(axis=-1)
    bm = oracle.pack_region_bitmap(ids, regions)
    assert bm.shape == (2, 3, 9, (regions + 31) // 32) and bm.dtype == np.int32
    words = bm.view(np.uint32)
    for idx in np.ndindex(ids.shape[:-1]):
        valid = {int(x) for x in ids[idx] if 0 <= x < regions}
        members = {w * 32 + b for w in range(words.shape[-1]) for b in range(32) if (int(words[idx][w]) >> b) & 1}
        assert members == valid
        assert sum(bin(int(w)).count("1") for w in words[idx]) == len(valid)


def test_order_and_repeats_do_not_matter():
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 500, size=(40, 60)).astype(np.int32)
    a = oracle.pack_region_bitmap(np.sort(ids, axis=-1), 500)
    b = oracle.pack_region_bitmap(ids, 500)
    c = oracle.pack_region_bitmap(np.concatenate([ids, ids[:, ::-1]], axis=-1), 500)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
