"""GPU parity of full-block CSR key masks (FlexAttention's from_kv_blocks
with a no-op mask_mod, "HF Attention Normalizers", "Important Limitations"):
the matrix-core kernels (bf16, query blocks of 128, key blocks of a multiple
of 64) and the per-row kernel (any block shape, f32), every row against the
oracle, with and without causal masking, head-shared and per-head lists,
query blocks without keys, and the entry-ignore rules."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
from oracle import attention_forward
from parity import TOL_OUT, compare_stats, _band

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _lists(rng, B, Hm, nqb, nkb, p, empty=True):
    num = np.zeros((B, Hm, nqb), dtype=np.int32)
    idx = np.full((B, Hm, nqb, nkb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hm):
            for r in range(nqb):
                c = np.nonzero(rng.random(nkb) < p)[0]
                num[b, h, r] = len(c)
                idx[b, h, r, :len(c)] = c
    if empty:
        num[0, 0, nqb // 2] = 0  # a query block without keys
    return num, idx


def _run(q, k, v, norm, causal, mask, scaling):
    num, idx, bq, bk = mask
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = torch.full((*q.shape[:3], 2), float("nan"), device="cuda")
    out, _ = apn.attn_fwd(qd, kd, vd, None, st, normalizer=norm, causal=causal, scaling=scaling,
                          block_mask=(torch.from_numpy(num).cuda(), torch.from_numpy(idx).cuda(),
                                      bq, bk))
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), st.double().cpu().numpy()


def _check(q, k, v, norm, causal, mask, scaling, where):
    out, st = _run(q, k, v, norm, causal, mask, scaling)
    B, Hq, Lq, D = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Lq)]
    o_ref, s_ref, det = attention_forward(q, k, v, norm, causal, 0, 0.0, scaling, rows=rows,
                                          return_probs=True, block_mask=mask)
    err = np.abs(out.reshape(-1, D) - o_ref).max()
    assert err <= TOL_OUT[q.dtype], f"{where} {norm}: out max-abs {err:.3e}"
    stg = st.reshape(-1, 2)
    for r, (b, h, i) in enumerate(rows):
        idx_, p, z = det[r]
        compare_stats(stg[r], s_ref[r], norm, len(idx_), _band(norm, z, s_ref[r][0]),
                      where=f"{where} {norm} row {(b, h, i)}")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,bk,causal,Hm", [
    (64, 128, True, 1),
    (64, 64, False, 4),
    (128, 128, False, 1),
    (128, 256, True, 4),
    (256, 64, True, 1)])
def test_matrix_core_path(norm, D, bk, causal, Hm):
    rng = np.random.default_rng(D + bk)
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 600, 700
    g = torch.Generator().manual_seed(D * 7 + bk)
    q = torch.randn(B, Hq, Lq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16)
    num, idx = _lists(rng, B, Hm, math.ceil(Lq / 128), math.ceil(Lk / bk), 0.4)
    _check(q, k, v, norm, causal, (num, idx, 128, bk), 1.0 / math.sqrt(D), f"mfma D{D} bk{bk}")


@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
def test_matrix_core_path_broad_scores(norm):
    # flat scores: the sparse kernel scores the listed tiles for block maxima
    # before collecting candidates
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 600, 700, 64
    g = torch.Generator().manual_seed(55)
    q = (0.5 * torch.randn(B, Hq, Lq, D, generator=g)).to(torch.bfloat16)
    k = (0.5 * torch.randn(B, Hkv, Lk, D, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16)
    num, idx = _lists(rng, B, 1, math.ceil(Lq / 128), math.ceil(Lk / 64), 0.6)
    _check(q, k, v, norm, True, (num, idx, 128, 64), 1.0 / math.sqrt(D), "broad scores")


@pytest.mark.parametrize("norm", NORMS)
def test_ignored_entries(norm):
    # repeated, descending and out-of-range entries are skipped like the oracle does
    B, Hq, Lq, Lk, D = 1, 2, 256, 512, 64
    g = torch.Generator().manual_seed(4)
    q, k, v = (torch.randn(B, n, L, D, generator=g).to(torch.bfloat16)
               for n, L in ((Hq, Lq), (1, Lk), (1, Lk)))
    num = np.array([[[5, 3]]], dtype=np.int32)
    idx = np.array([[[[1, 1, 0, 3, 9], [2, 3, -1, 0, 0]]]], dtype=np.int32)
    _check(q, k, v, norm, False, (num, idx, 128, 128), 0.125, "ignored entries")


@pytest.mark.parametrize("norm", NORMS)
def test_per_row_path_any_block_shape(norm):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, Lq, Lk, D, bq, bk = 2, 2, 1, 70, 90, 40, 16, 12
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, Hq, Lq, D, generator=g)
    k = torch.randn(B, Hkv, Lk, D, generator=g)
    v = torch.randn(B, Hkv, Lk, D, generator=g)
    num, idx = _lists(rng, B, Hq, math.ceil(Lq / bq), math.ceil(Lk / bk), 0.5)
    _check(q, k, v, norm, True, (num, idx, bq, bk), 0.3, "per-row")


@pytest.mark.parametrize("norm", NORMS)
def test_listing_every_block_is_bitwise_no_mask(norm):
    B, Hq, Hkv, L, D = 1, 4, 2, 1000, 128
    g = torch.Generator().manual_seed(21)
    q = torch.randn(B, Hq, L, D, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16).cuda()
    nqb, nkb = math.ceil(L / 128), math.ceil(L / 128)
    num = torch.full((B, 1, nqb), nkb, dtype=torch.int32, device="cuda")
    idx = torch.arange(nkb, dtype=torch.int32, device="cuda").expand(B, 1, nqb, nkb).contiguous()
    sa = torch.empty(B, Hq, L, 2, device="cuda")
    sb = torch.empty(B, Hq, L, 2, device="cuda")
    a, _ = apn.attn_fwd(q, k, v, None, sa, normalizer=norm, causal=True, scaling=0.09)
    b, _ = apn.attn_fwd(q, k, v, None, sb, normalizer=norm, causal=True, scaling=0.09,
                        block_mask=(num, idx, 128, 128))
    assert torch.equal(a, b) and torch.equal(sa, sb)
