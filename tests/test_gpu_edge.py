"""GPU parity: edge cases of the forward (empty and ragged inputs, Lq != Lk,
strided views, every head dim of the per-row path, paged caches)."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from parity import check_full, check_rows, gpu_fwd

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _rand(shape, seed, dtype=torch.float32, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lq,lk,causal,window", [(5, 1, True, 0), (1, 37, True, 0),
                                                 (9, 3, True, 0), (33, 33, True, 1),
                                                 (20, 70, False, 0), (70, 20, True, 7)])
def test_ragged_shapes(norm, dtype, lq, lk, causal, window):
    q = _rand((2, 6, lq, 24), 1, dtype)
    k = _rand((2, 3, lk, 24), 2, dtype)
    v = _rand((2, 3, lk, 24), 3, dtype)
    check_full(q, k, v, norm, causal, window, 0.0, 0.3, where=f"ragged {lq}x{lk}")


@pytest.mark.parametrize("norm", NORMS)
def test_no_keys(norm):
    q = _rand((1, 2, 4, 16), 4)
    k = torch.zeros(1, 2, 0, 16)
    out, st = gpu_fwd(q, k, k, norm, False, 0, 0.0, 0.25)
    assert (out == 0).all()
    want = {"softmax": (-math.inf, 0), "softmax1": (0, 1), "sparsemax": (math.inf, 0),
            "entmax15": (math.inf, 0)}[norm]
    assert (st[..., 0] == want[0]).all() and (st[..., 1] == want[1]).all()


def test_empty_batch_is_noop():
    q = torch.zeros(0, 2, 4, 16, device="cuda")
    out, _ = apn.attn_fwd(q, q, q, normalizer="softmax")
    torch.cuda.synchronize()
    assert out.shape == q.shape


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [1, 7, 32, 96, 200, 256])
def test_head_dims_f32(norm, D):
    q = _rand((1, 2, 13, D), 5)
    k = _rand((1, 1, 13, D), 6)
    v = _rand((1, 1, 13, D), 7)
    check_full(q, k, v, norm, True, 0, 0.0, 1.0 / math.sqrt(D), where=f"D={D}")


@pytest.mark.parametrize("norm", NORMS)
def test_strided_views(norm):
    # q as a [B, L, H, D] buffer viewed as [B, H, L, D]; k/v sliced from a wider buffer
    base = _rand((2, 19, 4, 32), 8)
    q = base.transpose(1, 2)
    kv = _rand((2, 2, 19, 64), 9)
    k, v = kv[..., :32], kv[..., 32:]
    qd = base.cuda().transpose(1, 2)
    kvd = kv.cuda()
    out = torch.empty(2, 4, 19, 32, device="cuda")
    st = torch.empty(2, 4, 19, 2, device="cuda")
    apn.attn_fwd(qd, kvd[..., :32], kvd[..., 32:], out, st, normalizer=norm, causal=True,
                 scaling=0.2)
    torch.cuda.synchronize()
    rows = [(b, h, i) for b in range(2) for h in range(4) for i in range(19)]
    check_rows(out.double().cpu().numpy(), st.double().cpu().numpy(), rows,
               q.contiguous(), k.contiguous(), v.contiguous(), norm, True, 0, 0.0, 0.2,
               where="strided")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_paged_small_per_row_path(norm, dtype):
    # Lq > 1 over a paged cache (chunked prefill shape), with NaN page tails
    cfg = W.PagedDecode("paged_small", 3, 4, 2, 40, "bf16" if dtype == torch.bfloat16 else "f32",
                        8, 3, 50, 0.2)
    x = W.make_paged(cfg)
    gq = torch.Generator().manual_seed(3)
    q = torch.randn(3, 4, 5, 40, generator=gq).to(dtype)
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
             "max_blocks": x.max_blocks}
    out, st = gpu_fwd(q, x.k_cache, x.v_cache, norm, True, 0, 0.0, 0.2, paged=paged)
    assert np.isfinite(out).all()
    rows = [(b, h, i) for b in range(3) for h in range(4) for i in range(5)]
    check_rows(out, st, rows, q, x.k_cache, x.v_cache, norm, True, 0, 0.0, 0.2, paged=paged,
               where="paged small")


def test_deterministic_repeat():
    q = _rand((1, 4, 40, 64), 11, torch.bfloat16)
    k = _rand((1, 2, 40, 64), 12, torch.bfloat16)
    for norm in NORMS:
        a = gpu_fwd(q, k, k, norm, True, 0, 0.0, 0.125)
        b = gpu_fwd(q, k, k, norm, True, 0, 0.0, 0.125)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("norm", NORMS)
def test_foreign_stream(norm):
    # a caller-supplied stream: outputs and the decode workspace the binding
    # allocates are tied to that stream; results equal the default stream's
    cfg = W.PagedDecode("dec_stream", 3, 8, 2, 128, "bf16", 16, 200, 1500, 0.09, seed=81)
    x = W.make_paged(cfg, device="cuda")
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens,
             "block_size": x.block_size, "max_blocks": x.max_blocks}
    ref, _ = apn.attn_fwd(x.q, x.k_cache, x.v_cache, normalizer=norm, causal=True,
                          scaling=cfg.scaling, paged=paged)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o, _ = apn.attn_fwd(x.q, x.k_cache, x.v_cache, normalizer=norm, causal=True,
                            scaling=cfg.scaling, paged=paged, stream=s.cuda_stream)
        outs.append(o)
        torch.empty(1 << 20, device="cuda").fill_(float("nan"))  # churn the caching allocator
    s.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
