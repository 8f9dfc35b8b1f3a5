"""Pins of the backward oracle (``oracle.backward``): PyTorch float64
autograd of independently written forwards (SDPA; the softcapped score path;
softmax1 as a softmax over the row extended by the sink logit with a zero
value), and central finite differences of the forward oracle for the sparse
normalizers.  CPU only."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward

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
