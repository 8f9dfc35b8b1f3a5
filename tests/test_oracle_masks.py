"""Pins for the oracle's mask: the page's worked example and closed-form counts."""

import os

import numpy as np
import pytest

from oracle import allowed_mask, kv_range

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden(name):
    shape = None
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# shape:"):
                shape = tuple(int(x) for x in line.split(":")[1].split())
            elif line and not line.startswith("#"):
                rows.append([c == "1" for c in line])
    return shape, np.array(rows, dtype=bool)


def test_worked_example_q6():
    """'tensorplay.nn.attention', create_mask(and_masks(causal, window<4)), 6x6."""
    shape, want = _load_golden("mask_causal_window4_q6.txt")
    got = allowed_mask(6, 6, causal=True, window=4)
    assert shape == (1, 1, 6, 6)
    assert got[None, None].shape == shape and got.dtype == np.bool_
    np.testing.assert_array_equal(got, want)
    assert int(got.sum()) == 18


def test_tiny_masked_q8():
    shape, want = _load_golden("mask_causal_window4_q8.txt")
    got = allowed_mask(8, 8, causal=True, window=4)
    np.testing.assert_array_equal(got, want)
    assert int(got.sum()) == 26


@pytest.mark.parametrize("L", [1, 5, 64, 333])
def test_causal_count(L):
    assert int(allowed_mask(L, L, causal=True).sum()) == L * (L + 1) // 2


@pytest.mark.parametrize("L,W", [(8, 4), (100, 7), (257, 64), (64, 64), (10, 1)])
def test_causal_window_count(L, W):
    # W(W+1)/2 pairs in the first W rows, then exactly W per row
    want = W * (W + 1) // 2 + (L - W) * W if L >= W else L * (L + 1) // 2
    assert int(allowed_mask(L, L, causal=True, window=W).sum()) == want


def test_unmasked_is_full():
    assert allowed_mask(3, 7, causal=False).all()


def test_bottom_right_alignment():
    # decode: one query against n keys sees all of them when causal
    m = allowed_mask(1, 9, causal=True)
    assert m.all()
    # the last query row always sees the last key; the first of 3 queries
    # against 5 keys sees keys 0..2
    m = allowed_mask(3, 5, causal=True)
    np.testing.assert_array_equal(m[0], [1, 1, 1, 0, 0])
    np.testing.assert_array_equal(m[2], [1, 1, 1, 1, 1])
    # more queries than keys: early queries see nothing
    m = allowed_mask(4, 2, causal=True)
    np.testing.assert_array_equal(m.sum(axis=1), [0, 0, 1, 2])


def test_window_decode_sees_last_w():
    m = allowed_mask(1, 10, causal=True, window=3)
    np.testing.assert_array_equal(np.nonzero(m[0])[0], [7, 8, 9])


def test_seq_len_limits_keys():
    m = allowed_mask(1, 10, causal=True, seq_len=6)
    np.testing.assert_array_equal(np.nonzero(m[0])[0], np.arange(6))


def test_window_without_causal_rejected():
    with pytest.raises(ValueError):
        allowed_mask(4, 4, causal=False, window=2)


@pytest.mark.parametrize("lq,lk,causal,window", [(8, 8, True, 4), (5, 13, True, 0),
                                                  (13, 5, True, 3), (6, 6, False, 0),
                                                  (1, 40, True, 16)])
def test_kv_range_matches_mask(lq, lk, causal, window):
    m = allowed_mask(lq, lk, causal, window)
    for i in range(lq):
        lo, hi = kv_range(i, lq, lk, causal, window)
        row = np.zeros(lk, dtype=bool)
        row[lo:hi] = True
        np.testing.assert_array_equal(row, m[i])
