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


# ---- full-block CSR masks ("HF Attention Normalizers", "Important Limitations")

from oracle import attention_forward  # noqa: E402
from oracle.masks import block_mask_allowed  # noqa: E402


def test_block_mask_entries_and_ignore_rules():
    # 5 queries in blocks of 3, 7 keys in blocks of 2 (4 key blocks)
    m = block_mask_allowed(5, 7, [4, 1], [[2, 2, 1, 5], [3, 0, 0, 0]], 3, 2)
    # q-block 0 uses 2 only: the repeated 2 and the 1 are not above their
    # predecessor, 5 is out of range
    expect = np.zeros((5, 7), dtype=bool)
    expect[0:3, 4:6] = True
    expect[3:5, 6] = True
    assert np.array_equal(m, expect)
    # counts clamp to [0, list length]
    assert not block_mask_allowed(3, 4, [-3], [[0, 1]], 3, 2).any()
    assert block_mask_allowed(3, 4, [9], [[0, 1]], 3, 2).all()


def _dense_blocks(rng, B, Hm, nqb, nkb, p):
    """Random block matrix and its CSR lists (ascending, padded with -1)."""
    blk = rng.random((B, Hm, nqb, nkb)) < p
    num = blk.sum(-1).astype(np.int32)
    idx = np.full((B, Hm, nqb, nkb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hm):
            for r in range(nqb):
                c = np.nonzero(blk[b, h, r])[0]
                idx[b, h, r, :len(c)] = c
    return blk, num, idx


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hm", [1, 4])
def test_block_mask_softmax_matches_sdpa(causal, Hm):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Lq, Lk, D, bq, bk = 2, 4, 2, 11, 13, 8, 4, 3
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    v = rng.standard_normal((B, Hkv, Lk, D))
    blk, num, idx = _dense_blocks(rng, B, Hm, -(-Lq // bq), -(-Lk // bk), 0.5)
    blk[0, 0, 0] = False  # one query block without keys
    num[0, 0, 0] = 0
    out, _ = attention_forward(q, k, v, "softmax", causal, 0, 0.0, 0.3,
                               block_mask=(num, idx, bq, bk))
    # independent construction: expand the block matrix with a Kronecker
    # product, crop, AND the bottom-right causal triangle; SDPA on it
    full = torch.kron(torch.from_numpy(blk.astype(np.float64)), torch.ones(bq, bk))[..., :Lq, :Lk] > 0
    if causal:
        full = full & torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
    full = full.expand(B, Hq, Lq, Lk) if Hm == 1 else full
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 1)
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kk, vv,
                                                           attn_mask=full, scale=0.3).numpy()
    has = full.any(-1).numpy()
    assert has.any() and (~has).any()
    np.testing.assert_allclose(out[has], ref[has], rtol=1e-12, atol=1e-12)
    assert (out[~has] == 0).all()  # a row without keys outputs zeros


@pytest.mark.parametrize("norm", ["softmax", "softmax1", "sparsemax", "entmax15"])
def test_block_mask_listing_every_block_is_no_mask(norm):
    rng = np.random.default_rng(8)
    B, Hq, Lq, Lk, D = 1, 2, 9, 10, 4
    q, k, v = (rng.standard_normal((B, Hq, n, D)) for n in (Lq, Lk, Lk))
    nqb, nkb = 3, 4
    num = np.full((B, 1, nqb), nkb, dtype=np.int32)
    idx = np.broadcast_to(np.arange(nkb, dtype=np.int32), (B, 1, nqb, nkb)).copy()
    a = attention_forward(q, k, v, norm, True, 0, 0.0, 0.7)
    b = attention_forward(q, k, v, norm, True, 0, 0.0, 0.7, block_mask=(num, idx, 3, 3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
