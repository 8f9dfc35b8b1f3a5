"""GPU parity of the bf16 prefill path (tiled matrix-core kernels for head
dims 64, 128, 256): reduced shapes compared in full, and the full workload
shapes compared on sampled rows, plus row-stat properties at full size."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from parity import check_full, check_rows, gpu_fwd, onehot_probe

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


# several 64-key tiles, a ragged tail, GQA 4:1, and q-blocks of 128 rows with a ragged end
@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("lq,lk,causal,window,cap", [
    (300, 300, True, 0, 0.0), (300, 300, False, 0, 0.0), (300, 300, True, 100, 0.0),
    (77, 300, True, 0, 0.0), (260, 260, True, 0, 30.0), (129, 129, True, 64, 10.0)],
    ids=["causal", "full", "window100", "lq77_lk300", "softcap30", "window64_cap10"])
def test_reduced(norm, D, lq, lk, causal, window, cap):
    q = _rand((2, 8, lq, D), 10 + D)
    k = _rand((2, 2, lk, D), 20 + D)
    v = _rand((2, 2, lk, D), 30 + D)
    check_full(q, k, v, norm, causal, window, cap, 1.0 / math.sqrt(D),
               where=f"D{D} {lq}x{lk} causal{causal} w{window} cap{cap}")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128])
def test_weight_pattern_probe(norm, D):
    # exact zeros where masked (and, for the sparse pair, off the support)
    q = _rand((1, 4, 200, D), 40, 2.0)
    k = _rand((1, 1, 200, D), 41, 2.0)
    for j0 in (0, 70, 130, 200 - D):
        onehot_probe(q, k, norm, True, 90, 0.0, 1.0 / math.sqrt(D), j0, where=f"probe D{D}")


@pytest.mark.parametrize("norm", NORMS)
def test_sigma_sweep_reduced(norm):
    # dense -> few keys, the support-size sweep of the Qwen3-shaped workload
    for sigma in (0.5, 1.0, 2.0):
        q = _rand((1, 4, 256, 128), 50, sigma)
        k = _rand((1, 2, 256, 128), 51, sigma)
        v = _rand((1, 2, 256, 128), 52)
        check_full(q, k, v, norm, True, 0, 0.0, 1.0 / math.sqrt(128), where=f"sigma{sigma}")


@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sigma", [0.4, 2.0])
def test_broad_and_peaked_scores(norm, D, sigma):
    # broad scores crowd the candidate buffers after the first key tile (the
    # workgroup then scores every tile for block maxima before collecting
    # candidates), peaked ones do not; several tiles, ragged ends, causal
    # and a window
    q = _rand((1, 4, 333, D), 60 + D, sigma)
    k = _rand((1, 2, 421, D), 61 + D, sigma)
    v = _rand((1, 2, 421, D), 62 + D)
    for window in (0, 150):
        check_full(q, k, v, norm, True, window, 0.0, 1.0 / math.sqrt(D),
                   where=f"sigma{sigma} D{D} window{window}")


def _sample_rows(cfg, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(cfg.B):
        for h in (0, cfg.Hq - 1):
            for i in (0, 1, 127, 128, cfg.Lq // 2, cfg.Lq - 1):
                rows.add((b, h, i))
    for _ in range(n_random):
        rows.add((int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq)), int(rng.integers(cfg.Lq))))
    return sorted(rows)


def _full_size(cfg, norm, n_random=24):
    q, k, v = W.make_prefill(cfg)
    out, st = gpu_fwd(q, k, v, norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling)
    assert np.isfinite(out).all()
    rows = _sample_rows(cfg, n_random, 7)
    check_rows(out, st, rows, q, k, v, norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling,
               where=cfg.name)
    return out, st


@pytest.mark.parametrize("norm", NORMS)
def test_llama_full_size(norm):
    _, st = _full_size(W.LLAMA, norm)
    if norm in ("sparsemax", "entmax15"):
        k = st[..., 1]
        assert (k >= 1).all() and (k <= np.arange(1, 2049)[None, None, :]).all()


@pytest.mark.parametrize("norm", ("softmax", "softmax1"))
def test_gemma_full_size(norm):
    _full_size(W.GEMMA, norm, n_random=16)


@pytest.mark.parametrize("sigma", W.QWEN_SIGMAS)
@pytest.mark.parametrize("norm", ("sparsemax", "entmax15", "softmax1"))
def test_qwen_full_size(norm, sigma):
    _, st = _full_size(W.qwen(sigma), norm, n_random=12)
    if norm != "softmax1":
        print(f"qwen sigma={sigma} {norm}: mean support {st[..., 1].mean():.2f}")


@pytest.mark.parametrize("lk", [65536, 65600])
@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
def test_sparse_long_key_range(norm, lk):
    # the sparse output pass gathers V rows through 16-bit key indices when
    # every key index fits them (lk <= 65536) and recomputes the scores tile
    # by tile otherwise; both sides of that boundary, keys near the far end
    # included (non-causal rows see every key; the last query rows are checked)
    lq = 40
    q = _rand((1, 2, lq, 64), 60, 2.0)
    k = _rand((1, 1, lk, 64), 61, 2.0)
    v = _rand((1, 1, lk, 64), 62)
    # make the last keys win for some rows: copy query rows into the far end
    k[0, 0, lk - 8:] = q[0, 0, :8] * 1.5
    out, st = gpu_fwd(q, k, v, norm, False, 0, 0.0, 0.125)
    rows = [(0, h, i) for h in range(2) for i in (0, 3, 7, 8, 20, lq - 1)]
    check_rows(out, st, rows, q, k, v, norm, False, 0, 0.0, 0.125, where=f"lk{lk}")
    assert (st[0, 0, :8, 1] >= 1).all()
