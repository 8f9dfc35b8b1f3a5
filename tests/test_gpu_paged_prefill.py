"""GPU parity of chunked prefill over a paged KV cache on the matrix-core
kernels (bf16, head dims 64/128/256, pages of a multiple of 8 keys; Lq > 1
queries align bottom-right against each sequence's own length): every row
against the oracle with NaN page tails, and bitwise equality with the same
sequence laid out in a contiguous cache (the tiles see identical operands)."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from parity import check_rows, gpu_fwd

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _paged(x):
    return {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
            "max_blocks": x.max_blocks}


def _chunk(cfg, Lq, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(cfg.B, cfg.Hq, Lq, cfg.D, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,Hq,Hkv,bs,lo,hi,Lq", [
    (64, 4, 2, 16, 40, 500, 96),    # some sequences shorter than the chunk (empty rows)
    (64, 2, 1, 8, 1, 300, 70),      # pages of 8: one transfer per page
    (128, 4, 2, 32, 150, 700, 130),
    (256, 4, 4, 16, 60, 400, 65)])
def test_all_rows(norm, D, Hq, Hkv, bs, lo, hi, Lq):
    cfg = W.PagedDecode(f"pchunk_{D}_{bs}", 3, Hq, Hkv, D, "bf16", bs, lo, hi, 1.0 / math.sqrt(D),
                        seed=400 + D + bs)
    x = W.make_paged(cfg)
    q = _chunk(cfg, Lq, 11 + D)
    out, st = gpu_fwd(q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling, paged=_paged(x))
    assert np.isfinite(out).all()  # no NaN page tail was read
    rows = [(b, h, i) for b in range(cfg.B) for h in range(Hq) for i in range(Lq)]
    check_rows(out, st, rows, q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling,
               paged=_paged(x), where=f"paged chunk D{D} bs{bs}")


@pytest.mark.parametrize("norm", NORMS)
def test_window_and_softcap(norm):
    cfg = W.PagedDecode("pchunk_wc", 2, 4, 2, 64, "bf16", 16, 200, 600, 0.125, seed=431)
    x = W.make_paged(cfg)
    q = _chunk(cfg, 80, 5)
    for window, cap in ((50, 0.0), (0, 20.0), (130, 30.0)):
        out, st = gpu_fwd(q, x.k_cache, x.v_cache, norm, True, window, cap, cfg.scaling,
                          paged=_paged(x))
        rows = [(b, h, i) for b in range(cfg.B) for h in range(cfg.Hq) for i in range(80)]
        check_rows(out, st, rows, q, x.k_cache, x.v_cache, norm, True, window, cap, cfg.scaling,
                   paged=_paged(x), where=f"paged chunk w{window} cap{cap}")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128])
def test_bitwise_equal_to_contiguous(norm, D):
    cfg = W.PagedDecode(f"pchunk_eq_{D}", 3, 8, 2, D, "bf16", 16, 300, 900, 1.0 / math.sqrt(D),
                        seed=77 + D)
    x = W.make_paged(cfg, device="cuda")
    Lq = 150
    q = _chunk(cfg, Lq, 3).cuda()
    out, st = apn.attn_fwd(q, x.k_cache, x.v_cache, None,
                           torch.empty(cfg.B, cfg.Hq, Lq, 2, device="cuda"), normalizer=norm,
                           causal=True, scaling=cfg.scaling, paged=_paged(x))
    lens = x.seq_lens.cpu().tolist()
    table = x.block_table.cpu()
    bs = x.block_size
    for b, n in enumerate(lens):
        pages = table[b, :(n + bs - 1) // bs].long().cuda()
        k = x.k_cache[pages].reshape(-1, cfg.Hkv, D)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        v = x.v_cache[pages].reshape(-1, cfg.Hkv, D)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        o1, s1 = apn.attn_fwd(q[b:b + 1].contiguous(), k, v, None,
                              torch.empty(1, cfg.Hq, Lq, 2, device="cuda"), normalizer=norm,
                              causal=True, scaling=cfg.scaling)
        assert torch.equal(o1[0], out[b]), f"{norm} D{D} sequence {b}: out differs"
        assert torch.equal(s1[0], st[b]), f"{norm} D{D} sequence {b}: row_stats differ"
