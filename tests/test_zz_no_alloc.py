"""attn_fwd_noalloc (no device allocation; the paged-decode workspace is the
library's fixed per-GPU scratch) against attn_fwd with a caller's workspace:
two calls in a row on the same scratch, the second on a smaller problem,
every normalizer; the kernels are the same, so the results are bitwise
equal.  A contiguous prefill (no workspace at all) as well."""

import math

import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _paged(x):
    return {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
            "max_blocks": x.max_blocks}


@pytest.mark.parametrize("norm", NORMS)
def test_noalloc_decode_matches_attn_fwd(norm):
    big = W.PagedDecode("noalloc_big", 8, 32, 8, 128, "bf16", 16, 1000, 6000,
                        1.0 / math.sqrt(128), seed=901)
    small = W.PagedDecode("noalloc_small", 3, 8, 2, 64, "bf16", 16, 50, 900, 0.125, seed=902)
    for cfg in (big, small):
        x = W.make_paged(cfg, device="cuda")
        paged = _paged(x)
        ref_st = torch.full((*x.q.shape[:3], 2), float("nan"), device="cuda")
        ref, _ = apn.attn_fwd(x.q, x.k_cache, x.v_cache, None, ref_st, normalizer=norm,
                              causal=True, scaling=cfg.scaling, paged=paged)
        out = torch.full_like(x.q, float("nan"))
        st = torch.full_like(ref_st, float("nan"))
        apn.attn_fwd_noalloc(x.q, x.k_cache, x.v_cache, out, st, normalizer=norm, causal=True,
                             scaling=cfg.scaling, paged=paged)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(out, ref), f"{cfg.name} {norm}: out differs"
        assert torch.equal(st, ref_st), f"{cfg.name} {norm}: row_stats differ"


def test_noalloc_prefill_matches_attn_fwd():
    g = torch.Generator().manual_seed(903)
    q = torch.randn(1, 4, 200, 64, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, 2, 200, 64, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, 200, 64, generator=g).to(torch.bfloat16).cuda()
    for norm in NORMS:
        ref, _ = apn.attn_fwd(q, k, v, normalizer=norm, causal=True, scaling=0.125)
        out = torch.empty_like(q)
        apn.attn_fwd_noalloc(q, k, v, out, normalizer=norm, causal=True, scaling=0.125)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), norm
