"""GPU parity of softmax1 with learned per-head sink logits (the virtual
key's logit b_h in place of 0) on every kernel family: tiled bf16 prefill
(head dims 64/128/256, causal, window, softcap), the per-row kernel (f32),
and paged split-KV decode."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from parity import check_rows, gpu_fwd

pytestmark = pytest.mark.gpu


def _sinks(hq, seed):
    # spread over large negative (sink irrelevant) to large positive (sink dominates)
    return np.random.default_rng(seed).uniform(-6.0, 6.0, size=hq).astype(np.float32)


@pytest.mark.parametrize("D,L,causal,window,cap", [
    (64, 200, True, 0, 0.0), (128, 160, True, 48, 0.0), (256, 96, True, 0, 30.0),
    (64, 130, False, 0, 0.0)])
def test_prefill_sinks(D, L, causal, window, cap):
    cfg = W.Prefill(f"sink{D}", 2, 8, 2, L, L, D, "bf16", causal, window, cap, 1.0 / math.sqrt(D),
                    seed=300 + D)
    q, k, v = W.make_prefill(cfg)
    sinks = _sinks(cfg.Hq, D)
    out, st = gpu_fwd(q, k, v, "softmax1", causal, window, cap, cfg.scaling, sinks=sinks)
    rows = [(b, h, i) for b in range(cfg.B) for h in range(cfg.Hq) for i in range(0, L, 7)]
    check_rows(out, st, rows, q, k, v, "softmax1", causal, window, cap, cfg.scaling,
               where=f"prefill sinks D{D}", sinks=sinks)


def test_generic_f32_sinks():
    cfg = W.Prefill("sink_f32", 1, 4, 2, 40, 40, 48, "f32", True, 0, 0.0, 0.2, seed=311)
    q, k, v = W.make_prefill(cfg)
    sinks = _sinks(cfg.Hq, 7)
    out, st = gpu_fwd(q, k, v, "softmax1", True, 0, 0.0, cfg.scaling, sinks=sinks)
    rows = [(0, h, i) for h in range(cfg.Hq) for i in range(cfg.Lq)]
    check_rows(out, st, rows, q, k, v, "softmax1", True, 0, 0.0, cfg.scaling,
               where="generic sinks", sinks=sinks)


def test_empty_rows_report_the_sink():
    # Lq > Lk with bottom-right causal alignment: the first rows see no key
    cfg = W.Prefill("sink_empty", 1, 4, 4, 24, 16, 64, "bf16", True, 0, 0.0, 0.125, seed=313)
    q, k, v = W.make_prefill(cfg)
    sinks = _sinks(cfg.Hq, 9)
    out, st = gpu_fwd(q, k, v, "softmax1", True, 0, 0.0, cfg.scaling, sinks=sinks)
    empty = cfg.Lq - cfg.Lk
    assert (out[:, :, :empty] == 0).all()
    np.testing.assert_allclose(st[0, :, :empty, 0], np.repeat(sinks[:, None], empty, 1), rtol=1e-6)
    assert (st[0, :, :empty, 1] == 1).all()


@pytest.mark.parametrize("D,Hq,Hkv,bs", [(128, 32, 8, 16), (64, 8, 2, 7)])
def test_decode_sinks(D, Hq, Hkv, bs):
    cfg = W.PagedDecode(f"dec_sink{D}", 4, Hq, Hkv, D, "bf16", bs, 1, 1300, 1.0 / math.sqrt(D),
                        seed=321)
    x = W.make_paged(cfg)
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
             "max_blocks": x.max_blocks}
    sinks = _sinks(Hq, 11)
    out, st = gpu_fwd(x.q, x.k_cache, x.v_cache, "softmax1", True, 0, 0.0, cfg.scaling,
                      paged=paged, sinks=sinks)
    rows = [(b, h, 0) for b in range(cfg.B) for h in range(Hq)]
    check_rows(out, st, rows, x.q, x.k_cache, x.v_cache, "softmax1", True, 0, 0.0, cfg.scaling,
               paged=paged, where=f"decode sinks D{D}", sinks=sinks)


def test_sinks_rejected_for_other_normalizers():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16, device="cuda")
    s = torch.zeros(2, dtype=torch.float32, device="cuda")
    for norm in ("softmax", "sparsemax", "entmax15"):
        with pytest.raises(apn.AttnError) as ei:
            apn.attn_fwd(q, q, q, normalizer=norm, causal=True, sinks=s)
        assert ei.value.status == apn.ATTN_E_INVALID
    with pytest.raises(ValueError):
        apn.attn_fwd(q, q, q, normalizer="softmax1", causal=True, sinks=s[:1])
