"""Pins for the oracle's attention forward (scores, GQA, mask, softcap, paging)."""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import allowed_mask, attention_forward, paged_attention_forward

NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


def _sdpa(q, k, v, mask, scaling):
    """PyTorch CPU fp64 SDPA with an explicit boolean mask and GQA."""
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    out = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.tensor(mask),
                                         scale=scaling, enable_gqa=True)
    return out.numpy()


def _brute_row(s_row, norm):
    """Weights of one row by definition: literal formulas, brute-force supports."""
    n = len(s_row)
    if n == 0:
        return []
    if norm == "softmax":
        e = [math.exp(x) for x in s_row]
        return [x / sum(e) for x in e]
    if norm == "softmax1":
        e = [math.exp(x) for x in s_row]
        return [x / (1.0 + sum(e)) for x in e]
    z = list(s_row) if norm == "sparsemax" else [x / 2.0 for x in s_row]
    power = 1 if norm == "sparsemax" else 2
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            zs = [z[i] for i in S]
            if power == 1:
                t = (sum(zs) - 1.0) / r
            else:
                mu = sum(zs) / r
                d = (1.0 - sum((x - mu) ** 2 for x in zs)) / r
                if d < 0:
                    continue
                t = mu - math.sqrt(d)
            if all(z[i] > t for i in S) and all(z[j] <= t for j in range(n) if j not in S):
                return [max(x - t, 0.0) ** power for x in z]
    raise AssertionError("no consistent support")


def _brute_attention(q, k, v, norm, causal, window, softcap, scaling):
    """Pure-Python loops over every index (tiny inputs only)."""
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Lq, D))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            for i in range(Lq):
                qp = i + Lk - Lq
                keys, svals = [], []
                for j in range(Lk):
                    if causal and j > qp:
                        continue
                    if window and qp - j >= window:
                        continue
                    s = 0.0
                    for d in range(D):
                        s += q[b, h, i, d] * k[b, kh, j, d]
                    s *= scaling
                    if softcap > 0:
                        s = softcap * math.tanh(s / softcap)
                    keys.append(j)
                    svals.append(s)
                p = _brute_row(svals, norm)
                for pj, j in zip(p, keys):
                    for d in range(D):
                        out[b, h, i, d] += pj * v[b, kh, j, d]
    return out


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("causal,window,softcap,lq,lk", [
    (False, 0, 0.0, 5, 5), (True, 0, 0.0, 5, 5), (True, 3, 0.0, 6, 6),
    (True, 0, 2.0, 3, 6), (True, 2, 1.5, 6, 4), (False, 0, 0.0, 2, 7)])
def test_against_brute_force_loops(norm, causal, window, softcap, lq, lk):
    # B=2, Hq=4, Hkv=2: exercises the GQA head map and both batch entries
    q = _rand((2, 4, lq, 3), 11, 1.5)
    k = _rand((2, 2, lk, 3), 12, 1.5)
    v = _rand((2, 2, lk, 3), 13)
    out, _ = attention_forward(q, k, v, norm, causal, window, softcap, 0.7)
    want = _brute_attention(q, k, v, norm, causal, window, softcap, 0.7)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal,window,lq,lk", [(False, 0, 9, 9), (True, 0, 16, 16),
                                                  (True, 5, 16, 16), (True, 0, 4, 19)])
def test_softmax_matches_torch_sdpa_gqa(causal, window, lq, lk):
    q = _rand((2, 6, lq, 8), 1)
    k = _rand((2, 2, lk, 8), 2)
    v = _rand((2, 2, lk, 8), 3)
    mask = allowed_mask(lq, lk, causal, window)
    out, stats = attention_forward(q, k, v, "softmax", causal, window, 0.0, 0.3)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask, 0.3), rtol=1e-12, atol=1e-13)
    # row stats: log-sum-exp of the allowed scores
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, np.repeat(k, 3, axis=1))
    s = np.where(mask, s, -np.inf)
    lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    np.testing.assert_allclose(stats[..., 0] + np.log(stats[..., 1]), lse, rtol=1e-12)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 4)])
def test_softmax1_is_sdpa_with_zero_sink(causal, window):
    # softmax1 equals plain attention with one extra key k=0, v=0 that every
    # query sees ("HF Attention Normalizers", "Important Limitations")
    lq = lk = 12
    q = _rand((1, 4, lq, 8), 4, 2.0)
    k = _rand((1, 2, lk, 8), 5, 2.0)
    v = _rand((1, 2, lk, 8), 6)
    out, stats = attention_forward(q, k, v, "softmax1", causal, window, 0.0, 0.5)
    k1 = np.concatenate([np.zeros((1, 2, 1, 8)), k], axis=2)
    v1 = np.concatenate([np.zeros((1, 2, 1, 8)), v], axis=2)
    mask = np.concatenate([np.ones((lq, 1), bool), allowed_mask(lq, lk, causal, window)], 1)
    np.testing.assert_allclose(out, _sdpa(q, k1, v1, mask, 0.5), rtol=1e-12, atol=1e-13)
    assert (stats[..., 0] >= 0).all()


def test_softcap_on_known_scores():
    # choose raw scores whose capped values are known, c_j = cap * tanh(s_j / cap):
    # s_j = cap * atanh(c_j / cap).  One head dim, q = 1, k_j = s_j.
    cap = 5.0
    c = np.array([-4.0, -1.0, 0.0, 2.5, 4.9])
    s = cap * np.arctanh(c / cap)
    q = np.ones((1, 1, 1, 1))
    k = s.reshape(1, 1, -1, 1)
    v = _rand((1, 1, 5, 1), 9)
    out, _ = attention_forward(q, k, v, "softmax", False, 0, cap, 1.0)
    want = _sdpa(q, c.reshape(1, 1, -1, 1), v, np.ones((1, 5), bool), 1.0)
    np.testing.assert_allclose(out, want, rtol=1e-12)


def test_softcap_bounds_and_limit():
    q = _rand((1, 2, 6, 4), 21, 10.0)
    k = _rand((1, 2, 6, 4), 22, 10.0)
    v = _rand((1, 2, 6, 4), 23)
    for norm in NORMS:
        a, _ = attention_forward(q, k, v, norm, True, 0, 1e9, 0.5)
        b, _ = attention_forward(q, k, v, norm, True, 0, 0.0, 0.5)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)
    # with a cap of 1 every capped score lies in (-1, 1): softmax weights of a row
    # can differ by at most a factor e^2 (reached when tanh saturates in fp64)
    _, _, p = attention_forward(q, k, v, "softmax", False, 0, 1.0, 0.5, return_probs=True)
    assert (p.max(-1) / p.min(-1) <= math.exp(2.0) * (1 + 1e-12)).all()


def test_gqa_equals_expanded_heads():
    q = _rand((1, 8, 7, 5), 31)
    k = _rand((1, 2, 7, 5), 32)
    v = _rand((1, 2, 7, 5), 33)
    for norm in NORMS:
        a, sa = attention_forward(q, k, v, norm, True, 0, 0.0, 0.4)
        kx = np.repeat(k, 4, axis=1)  # head h -> kv head h // 4
        vx = np.repeat(v, 4, axis=1)
        b, sb = attention_forward(q, kx, vx, norm, True, 0, 0.0, 0.4)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(sa, sb)


def test_fully_masked_rows_are_zero():
    q = _rand((1, 2, 4, 3), 41)
    k = _rand((1, 2, 2, 3), 42)
    v = _rand((1, 2, 2, 3), 43)
    for norm, st in (("softmax", (-math.inf, 0)), ("softmax1", (0, 1)),
                     ("sparsemax", (math.inf, 0)), ("entmax15", (math.inf, 0))):
        out, stats = attention_forward(q, k, v, norm, True, 0, 0.0, 1.0)
        assert (out[:, :, :2] == 0).all()
        assert (stats[:, :, :2, 0] == st[0]).all() and (stats[:, :, :2, 1] == st[1]).all()


def test_rows_subset_matches_full():
    q = _rand((2, 4, 9, 6), 51)
    k = _rand((2, 2, 9, 6), 52)
    v = _rand((2, 2, 9, 6), 53)
    rows = [(0, 0, 0), (1, 3, 8), (0, 2, 4), (1, 1, 5)]
    for norm in NORMS:
        full, fs = attention_forward(q, k, v, norm, True, 3, 0.0, 0.5)
        sub, ss = attention_forward(q, k, v, norm, True, 3, 0.0, 0.5, rows=rows)
        for r, (b, h, i) in enumerate(rows):
            # a one-row matmul may round differently from a block matmul
            np.testing.assert_allclose(sub[r], full[b, h, i], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(ss[r], fs[b, h, i], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- paged

def _scatter_to_pages(k, lens, bs, seed):
    """Build a paged cache from contiguous keys [B,Hkv,L,D] (test-side scatter)."""
    B, Hkv, L, D = k.shape
    pages = [(n + bs - 1) // bs for n in lens]
    nb = sum(pages)
    perm = np.random.default_rng(seed).permutation(nb)
    cache = np.full((nb, bs, Hkv, D), np.nan)
    table = -np.ones((B, max(pages)), dtype=np.int64)
    off = 0
    for b in range(B):
        for j in range(pages[b]):
            table[b, j] = perm[off + j]
        off += pages[b]
        for t in range(lens[b]):
            cache[table[b, t // bs], t % bs] = k[b, :, t]
    return cache, table


@pytest.mark.parametrize("norm", NORMS)
def test_paged_equals_contiguous(norm):
    B, Hq, Hkv, D, bs = 3, 4, 2, 5, 4
    lens = [7, 12, 1]
    L = max(lens)
    q = _rand((B, Hq, 1, D), 61)
    k = _rand((B, Hkv, L, D), 62)
    v = _rand((B, Hkv, L, D), 63)
    kc, table = _scatter_to_pages(k, lens, bs, 64)
    vc, _ = _scatter_to_pages(v, lens, bs, 64)
    out, st = paged_attention_forward(q, kc, vc, table, lens, norm, causal=True)
    assert np.isfinite(out).all()  # the NaN page tails were never read
    for b in range(B):
        n = lens[b]
        want, wst = attention_forward(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], norm,
                                      True, 0, 0.0, 1 / math.sqrt(D))
        np.testing.assert_allclose(out[b], want[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(st[b], wst[0], rtol=1e-13)


def test_paged_permutation_invariance():
    B, Hq, Hkv, D, bs = 2, 2, 1, 4, 3
    lens = [8, 5]
    q = _rand((B, Hq, 1, D), 71)
    k = _rand((B, Hkv, 8, D), 72)
    v = _rand((B, Hkv, 8, D), 73)
    a = paged_attention_forward(q, *[_scatter_to_pages(x, lens, bs, 1)[0] for x in (k, v)],
                                _scatter_to_pages(k, lens, bs, 1)[1], lens, "sparsemax")
    b = paged_attention_forward(q, *[_scatter_to_pages(x, lens, bs, 2)[0] for x in (k, v)],
                                _scatter_to_pages(k, lens, bs, 2)[1], lens, "sparsemax")
    np.testing.assert_array_equal(a[0], b[0])


def test_workload_paged_generator_small():
    cfg = W.PagedDecode("small", 3, 4, 2, 8, "bf16", 16, 5, 40, 0.35)
    x = W.make_paged(cfg)
    lens = x.seq_lens.tolist()
    for norm in NORMS:
        out, st = paged_attention_forward(x.q, x.k_cache, x.v_cache, x.block_table.numpy(),
                                          lens, norm, scaling=0.35)
        assert np.isfinite(out).all()


def test_tiny_workload_runs():
    q, k, v = W.make_prefill(W.TINY)
    assert q.dtype == torch.float32 and q.shape == (1, 2, 8, 16)
    for norm in NORMS:
        for causal, window in ((False, 0), (True, 4)):
            out, st = attention_forward(q, k, v, norm, causal, window, 0.0, 0.25)
            assert np.isfinite(out).all()


@pytest.mark.parametrize("causal,window,softcap", [(False, 0, 0.0), (True, 0, 0.0), (True, 4, 3.0)])
def test_learned_sinks_are_sdpa_with_a_biased_zero_key(causal, window, softcap):
    # a learned sink b_h is one extra key of value 0 whose logit is b_h for
    # every query ("Attention variants: what to open up, and how far", "What
    # cannot be drawn today"): SDPA with a zero key and an additive float mask
    # that puts b_h on that key's column and -inf on masked keys
    lq = lk = 10
    q = _rand((1, 4, lq, 8), 14, 1.5)
    k = _rand((1, 2, lk, 8), 15, 1.5)
    v = _rand((1, 2, lk, 8), 16)
    sinks = np.array([-1.5, 0.0, 0.7, 3.0])
    out, stats = attention_forward(q, k, v, "softmax1", causal, window, softcap, 0.5, sinks=sinks)
    allowed = allowed_mask(lq, lk, causal, window)
    # scores with softcap applied, as the reference of the real keys
    s = 0.5 * np.einsum("hid,hjd->hij", q[0], np.repeat(k[0], 2, axis=0))
    if softcap:
        s = softcap * np.tanh(s / softcap)
    bias = np.where(allowed[None], s, -np.inf)                                  # [4, lq, lk]
    bias = np.concatenate([np.broadcast_to(sinks[:, None, None], (4, lq, 1)), bias], axis=2)
    v1 = np.concatenate([np.zeros((1, 2, 1, 8)), v], axis=2)
    # scores come entirely from the float mask: zero queries and keys
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    want = F.scaled_dot_product_attention(t(np.zeros((1, 4, lq, 8))), t(np.zeros((1, 2, lk + 1, 8))),
                                          t(v1), attn_mask=t(bias[None]), enable_gqa=True).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)
    # m = max(b, max s) per row
    assert (stats[..., 0] >= sinks[None, :, None] - 1e-15).all()


def test_learned_sink_limits():
    q = _rand((1, 2, 6, 8), 17)
    k = _rand((1, 1, 6, 8), 18)
    v = _rand((1, 1, 6, 8), 19)
    o_sm, _ = attention_forward(q, k, v, "softmax", True, 0, 0.0, 0.4)
    o_far, _ = attention_forward(q, k, v, "softmax1", True, 0, 0.0, 0.4, sinks=[-800.0, -800.0])
    np.testing.assert_allclose(o_far, o_sm, rtol=1e-13, atol=1e-15)
    o_s1, st_s1 = attention_forward(q, k, v, "softmax1", True, 0, 0.0, 0.4)
    o_z, st_z = attention_forward(q, k, v, "softmax1", True, 0, 0.0, 0.4, sinks=[0.0, 0.0])
    assert np.array_equal(o_s1, o_z) and np.array_equal(st_s1, st_z)
    with pytest.raises(ValueError):
        attention_forward(q, k, v, "softmax", True, 0, 0.0, 0.4, sinks=[0.0, 0.0])


def test_varlen_equals_padded_batch_sdpa():
    # packed requests with their own lengths (Lq <= Lk, bottom-right causal)
    # against PyTorch SDPA on a zero-padded batch with an explicit mask
    from oracle import varlen_attention_forward
    lq = [3, 0, 7, 1, 5]
    lk = [5, 2, 7, 4, 9]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    Hq, Hkv, D = 4, 2, 8
    q = _rand((cq[-1], Hq, D), 21)
    k = _rand((ck[-1], Hkv, D), 22)
    v = _rand((ck[-1], Hkv, D), 23)
    out, st = varlen_attention_forward(q, k, v, cq, ck, "softmax", True, 3, 0.0, 0.4)
    B, Lq, Lk = len(lq), max(lq), max(lk)
    qp = np.zeros((B, Hq, Lq, D)); kp = np.zeros((B, Hkv, Lk, D)); vp = np.zeros((B, Hkv, Lk, D))
    mask = np.zeros((B, 1, Lq, Lk), bool)
    for r in range(B):
        qp[r, :, :lq[r]] = np.transpose(q[cq[r]:cq[r + 1]], (1, 0, 2))
        kp[r, :, :lk[r]] = np.transpose(k[ck[r]:ck[r + 1]], (1, 0, 2))
        vp[r, :, :lk[r]] = np.transpose(v[ck[r]:ck[r + 1]], (1, 0, 2))
        for i in range(lq[r]):
            for j in range(lk[r]):
                qpos = i + lk[r] - lq[r]
                mask[r, 0, i, j] = j <= qpos and qpos - j < 3
    mask[..., 0] |= ~mask.any(-1)  # keep SDPA defined on padded rows (ignored)
    want = _sdpa(qp, kp, vp, mask, 0.4)
    for r in range(B):
        got = np.transpose(out[cq[r]:cq[r + 1]], (1, 0, 2))
        np.testing.assert_allclose(got, want[r, :, :lq[r]], rtol=1e-12, atol=1e-13)
