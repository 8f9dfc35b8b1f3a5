"""Pins of the backward oracle (``oracle.backward``): PyTorch float64
autograd of independently written forwards (SDPA; the softcapped score path;
softmax1 as a softmax over the row extended by the sink logit with a zero
value), and central finite differences of the forward oracle for the sparse
normalizers.  CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward, varlen_attention_backward,
                    varlen_attention_forward)

NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _inputs(seed, B=1, Hq=4, Hkv=2, Lq=7, Lk=9, D=5):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, Hq, Lq, D)), g.standard_normal((B, Hkv, Lk, D)),
            g.standard_normal((B, Hkv, Lk, D)), g.standard_normal((B, Hq, Lq, D)))


def _bool_mask(Lq, Lk, causal, window):
    i = torch.arange(Lq)[:, None] + (Lk - Lq)
    j = torch.arange(Lk)[None, :]
    m = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window:
        m &= i - j < window
    return m


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_softmax_matches_sdpa_autograd(causal, window):
    q, k, v, do = _inputs(1)
    G = q.shape[1] // k.shape[1]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _bool_mask(q.shape[2], k.shape[2], causal, window)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), attn_mask=mask, scale=0.4)
    out.backward(torch.tensor(do))
    dq, dk, dv, _ = attention_backward(q, k, v, do, "softmax", causal, window, 0.0, 0.4)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)


def test_softcap_matches_autograd_of_the_score_path():
    q, k, v, do = _inputs(2)
    G = q.shape[1] // k.shape[1]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = 0.7 * tq @ tk.repeat_interleave(G, 1).transpose(-1, -2)
    s = 2.5 * torch.tanh(s / 2.5)
    s = s.masked_fill(~_bool_mask(q.shape[2], k.shape[2], True, 0), float("-inf"))
    out = torch.softmax(s, -1) @ tv.repeat_interleave(G, 1)
    out.backward(torch.tensor(do))
    dq, dk, dv, _ = attention_backward(q, k, v, do, "softmax", True, 0, 2.5, 0.7)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)


def test_softmax1_sinks_match_extended_row_autograd():
    q, k, v, do = _inputs(3)
    Hq, Lq, Lk = q.shape[1], q.shape[2], k.shape[2]
    G = Hq // k.shape[1]
    sinks = np.array([0.3, -1.0, 2.0, 0.0])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tb = torch.tensor(sinks, requires_grad=True)
    s = 0.5 * tq @ tk.repeat_interleave(G, 1).transpose(-1, -2)
    s = s.masked_fill(~_bool_mask(Lq, Lk, True, 0), float("-inf"))
    ext = torch.cat([s, tb.view(1, Hq, 1, 1).expand(1, Hq, Lq, 1)], -1)
    vext = torch.cat([tv.repeat_interleave(G, 1), torch.zeros(1, Hq, 1, q.shape[3],
                                                            dtype=torch.float64)], 2)
    out = torch.softmax(ext, -1) @ vext
    out.backward(torch.tensor(do))
    dq, dk, dv, dsinks = attention_backward(q, k, v, do, "softmax1", True, 0, 0.0, 0.5,
                                            sinks=sinks)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (dsinks, tb.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)


def _loss(q, k, v, do, norm, causal, window, cap, scaling):
    out, _ = attention_forward(q, k, v, norm, causal, window, cap, scaling)
    return float((out * do).sum())


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("causal,window,cap", [(False, 0, 0.0), (True, 3, 0.0), (True, 0, 3.0)])
def test_finite_differences(norm, causal, window, cap):
    # central differences of <out, dO> against the analytic gradients; the
    # scale puts several keys in the sparse supports, and the step is far
    # below the distance of any score to tau (support fixed in the stencil)
    q, k, v, do = _inputs(7, Hq=2, Hkv=1, Lq=5, Lk=6, D=3)
    scaling = 0.6
    dq, dk, dv, _ = attention_backward(q, k, v, do, norm, causal, window, cap, scaling)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = x[ix]
            x[ix] = old + eps
            fp = _loss(q, k, v, do, norm, causal, window, cap, scaling)
            x[ix] = old - eps
            fm = _loss(q, k, v, do, norm, causal, window, cap, scaling)
            x[ix] = old
            num[ix] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-5, atol=1e-7)


def test_sparse_gradients_vanish_off_the_support():
    # a key outside every row's support moves nothing: its dK and dV are 0
    q, k, v, do = _inputs(9, Hq=2, Hkv=1, Lq=4, Lk=12, D=3)
    for norm in ("sparsemax", "entmax15"):
        _, _, probs = attention_forward(q, k, v, norm, False, 0, 0.0, 4.0, return_probs=True)
        dead = np.nonzero(~(probs[0] > 0).any(axis=(0, 1)))[0]
        assert dead.size > 0
        _, dk, dv, _ = attention_backward(q, k, v, do, norm, False, 0, 0.0, 4.0)
        assert np.all(dk[0, 0, dead] == 0) and np.all(dv[0, 0, dead] == 0)


def _blocks(rng, B, Hm, nqb, nkb, p):
    """A random block matrix and its CSR lists (ascending block indices)."""
    blk = rng.random((B, Hm, nqb, nkb)) < p
    num = blk.sum(-1).astype(np.int64)
    idx = np.full((B, Hm, nqb, nkb), -1, dtype=np.int64)
    for b in range(B):
        for h in range(Hm):
            for r in range(nqb):
                c = np.nonzero(blk[b, h, r])[0]
                idx[b, h, r, :len(c)] = c
    return blk, num, idx


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hm", [1, 4])
def test_block_mask_softmax_matches_sdpa_autograd(causal, Hm):
    # the block mask expanded by a Kronecker product and cropped, ANDed with
    # the bottom-right causal triangle, through SDPA's autograd
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Lq, Lk, D, bq, bk = 2, 4, 2, 11, 13, 5, 4, 3
    q, k, v, do = (rng.standard_normal(s) for s in
                   ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D), (B, Hq, Lq, D)))
    blk, num, idx = _blocks(rng, B, Hm, -(-Lq // bq), -(-Lk // bk), 0.6)
    blk[0, 0, 1] = False  # a query block without keys
    num[0, 0, 1] = 0
    full = torch.kron(torch.from_numpy(blk.astype(np.float64)), torch.ones(bq, bk))[..., :Lq, :Lk] > 0
    if causal:
        full = full & torch.ones(Lq, Lk, dtype=torch.bool).tril(Lk - Lq)
    full = full.expand(B, Hq, Lq, Lk) if Hm == 1 else full
    G = Hq // Hkv
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = 0.45 * tq @ tk.repeat_interleave(G, 1).transpose(-1, -2)
    w = torch.softmax(s.masked_fill(~full, float("-inf")), -1)
    w = torch.nan_to_num(w, nan=0.0)  # rows without keys: no weights
    (w @ tv.repeat_interleave(G, 1)).backward(torch.tensor(do))
    dq, dk, dv, _ = attention_backward(q, k, v, do, "softmax", causal, 0, 0.0, 0.45,
                                       block_mask=(num, idx, bq, bk))
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("norm", NORMS)
def test_block_mask_finite_differences(norm):
    rng = np.random.default_rng(12)
    q, k, v, do = _inputs(13, Hq=2, Hkv=1, Lq=6, Lk=7, D=3)
    blk, num, idx = _blocks(rng, 1, 2, 3, 3, 0.7)
    bm = (num, idx, 2, 3)
    scaling = 0.6
    dq, dk, dv, _ = attention_backward(q, k, v, do, norm, True, 0, 0.0, scaling, block_mask=bm)

    def loss(q_, k_, v_):
        out, _ = attention_forward(q_, k_, v_, norm, True, 0, 0.0, scaling, block_mask=bm)
        return float((out * do).sum())
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num_g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = x[ix]
            x[ix] = old + eps
            fp = loss(q, k, v)
            x[ix] = old - eps
            fm = loss(q, k, v)
            x[ix] = old
            num_g[ix] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num_g, rtol=1e-5, atol=1e-7)


def _packed(seed, q_lens, k_lens, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    tq, tk = sum(q_lens), sum(k_lens)
    cu = lambda lens: np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (g.standard_normal((tq, Hq, D)), g.standard_normal((tk, Hkv, D)),
            g.standard_normal((tk, Hkv, D)), g.standard_normal((tq, Hq, D)), cu(q_lens),
            cu(k_lens))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_varlen_softmax_matches_padded_batch_autograd(causal, window):
    # each request zero-padded into a batch entry of its own; SDPA autograd
    # with the padding masked; gradients of the real tokens compared
    q_lens, k_lens = (3, 5, 1, 4), (6, 5, 2, 7)
    Hq, Hkv, D = 4, 2, 5
    q, k, v, do, cq, ck = _packed(21, q_lens, k_lens, Hq, Hkv, D)
    R, Lq, Lk = len(q_lens), max(q_lens), max(k_lens)
    G = Hq // Hkv
    Q = torch.zeros(R, Hq, Lq, D, dtype=torch.float64)
    K = torch.zeros(R, Hkv, Lk, D, dtype=torch.float64)
    V = torch.zeros(R, Hkv, Lk, D, dtype=torch.float64)
    DO = torch.zeros(R, Hq, Lq, D, dtype=torch.float64)
    mask = torch.zeros(R, 1, Lq, Lk, dtype=torch.bool)
    for r in range(R):
        nq, nk = q_lens[r], k_lens[r]
        Q[r, :, :nq] = torch.from_numpy(q[cq[r]:cq[r + 1]]).transpose(0, 1)
        K[r, :, :nk] = torch.from_numpy(k[ck[r]:ck[r + 1]]).transpose(0, 1)
        V[r, :, :nk] = torch.from_numpy(v[ck[r]:ck[r + 1]]).transpose(0, 1)
        DO[r, :, :nq] = torch.from_numpy(do[cq[r]:cq[r + 1]]).transpose(0, 1)
        i = torch.arange(nq)[:, None] + (nk - nq)  # bottom-right aligned query positions
        j = torch.arange(nk)[None, :]
        m = torch.ones(nq, nk, dtype=torch.bool)
        if causal:
            m &= j <= i
        if window:
            m &= i - j < window
        mask[r, 0, :nq, :nk] = m
    for t in (Q, K, V):
        t.requires_grad_(True)
    s = 0.35 * Q @ K.repeat_interleave(G, 1).transpose(-1, -2)
    w = torch.nan_to_num(torch.softmax(s.masked_fill(~mask, float("-inf")), -1), nan=0.0)
    (w @ V.repeat_interleave(G, 1)).backward(DO)
    dq, dk, dv, _ = varlen_attention_backward(q, k, v, do, cq, ck, "softmax", causal, window,
                                              0.0, 0.35)
    for r in range(R):
        nq, nk = q_lens[r], k_lens[r]
        np.testing.assert_allclose(dq[cq[r]:cq[r + 1]], Q.grad[r, :, :nq].transpose(0, 1).numpy(),
                                   rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dk[ck[r]:ck[r + 1]], K.grad[r, :, :nk].transpose(0, 1).numpy(),
                                   rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv[ck[r]:ck[r + 1]], V.grad[r, :, :nk].transpose(0, 1).numpy(),
                                   rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("norm", NORMS)
def test_varlen_finite_differences(norm):
    q_lens, k_lens = (2, 3), (4, 3)
    q, k, v, do, cq, ck = _packed(22, q_lens, k_lens, 2, 1, 3)
    scaling = 0.7
    dq, dk, dv, _ = varlen_attention_backward(q, k, v, do, cq, ck, norm, True, 0, 0.0, scaling)

    def loss(q_, k_, v_):
        out, _ = varlen_attention_forward(q_, k_, v_, cq, ck, norm, True, 0, 0.0, scaling)
        return float((out * do).sum())
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num_g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = x[ix]
            x[ix] = old + eps
            fp = loss(q, k, v)
            x[ix] = old - eps
            fm = loss(q, k, v)
            x[ix] = old
            num_g[ix] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num_g, rtol=1e-5, atol=1e-7)
