"""Every workload shape that bench.py measures takes the tiled matrix-core
prefill or the split-KV decode kernels, never the per-row correctness path
(the kernel family is a fixed function of the arguments: attn_fwd_path)."""

import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [W.LLAMA, W.qwen(0.5), W.qwen(1.0), W.qwen(2.0), W.GEMMA],
                         ids=lambda c: c.name)
def test_prefill_workloads_take_the_matrix_cores(cfg):
    q, k, v = (x.cuda() for x in W.make_prefill(cfg))
    out = torch.empty_like(q)
    for norm in cfg.normalizers:
        assert apn.attn_fwd_path(q, k, v, out, normalizer=norm, causal=cfg.causal,
                                 window=cfg.window, softcap=cfg.softcap,
                                 scaling=cfg.scaling) == "prefill_mfma", norm
    if cfg is W.LLAMA:
        for norm in cfg.normalizers:
            assert apn.attn_bwd_path(q, k, v, out, normalizer=norm, causal=True,
                                     scaling=cfg.scaling, out=out) == "bwd_mfma", norm


def test_paged_workload_paths():
    cfg = W.DECODE
    x = W.make_paged(cfg, device="cuda")
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
             "max_blocks": x.max_blocks}
    chunk = torch.empty(cfg.B, cfg.Hq, 512, cfg.D, dtype=torch.bfloat16, device="cuda")
    for norm in cfg.normalizers:
        assert apn.attn_fwd_path(x.q, x.k_cache, x.v_cache, normalizer=norm, causal=True,
                                 scaling=cfg.scaling, paged=paged) == "decode_split", norm
        assert apn.attn_fwd_path(chunk, x.k_cache, x.v_cache, normalizer=norm, causal=True,
                                 scaling=cfg.scaling, paged=paged) == "prefill_mfma", norm
