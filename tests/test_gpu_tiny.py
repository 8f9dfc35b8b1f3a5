"""GPU parity: the tiny f32 workload (B=1, H=2, L=8, head_dim=16), every
normalizer, unmasked and causal AND window(q - k < 4), through the C ABI."""

import pytest
import torch

import workloads as W
from parity import check_full, onehot_probe

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("cfg", [W.TINY, W.TINY_MASKED], ids=["unmasked", "causal_window4"])
def test_tiny(norm, cfg):
    q, k, v = W.make_prefill(cfg)
    check_full(q, k, v, norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling, where=cfg.name)
    # Lk = 8 <= head_dim = 16: one probe recovers every weight
    onehot_probe(q, k, norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling, 0, where=cfg.name)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 4)])
def test_tiny_q_equals_k_equals_v(norm, causal, window):
    # the SDPA example passes one tensor as q, k and v ("tensorplay.nn.attention")
    x = torch.randn(1, 2, 8, 16, generator=torch.Generator().manual_seed(1001))
    check_full(x, x, x, norm, causal, window, 0.0, 0.25, where="q=k=v")
    onehot_probe(x, x, norm, causal, window, 0.0, 0.25, 0, where="q=k=v")


@pytest.mark.parametrize("norm", NORMS)
def test_tiny_softcap_and_gqa_f32(norm):
    g = torch.Generator().manual_seed(7)
    q = torch.randn(2, 4, 11, 16, generator=g) * 3
    k = torch.randn(2, 2, 11, 16, generator=g) * 3
    v = torch.randn(2, 2, 11, 16, generator=g)
    check_full(q, k, v, norm, True, 5, 2.5, 0.25, where="softcap+gqa")
