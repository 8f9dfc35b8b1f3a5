"""GPU parity of the paged split-KV decode path (bf16, one query token per
sequence, head dims 64/128/256): every row of reduced batches, invariants of
the paging and splitting, and sampled rows of the full decode workload."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from oracle import paged_attention_forward
from parity import check_rows, gpu_fwd

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _paged(x):
    return {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
            "max_blocks": x.max_blocks}


def _run(cfg, norm, window=0, softcap=0.0, x=None):
    x = x or W.make_paged(cfg)
    out, st = gpu_fwd(x.q, x.k_cache, x.v_cache, norm, True, window, softcap, cfg.scaling,
                      paged=_paged(x))
    return x, out, st


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,Hq,Hkv,bs,lo,hi", [
    (128, 32, 8, 16, 1, 1500),     # the decode workload's head layout, short sequences
    (64, 8, 8, 16, 600, 1100),     # G = 1, several splits
    (256, 16, 2, 32, 30, 700),     # G = 8, larger pages
    (128, 12, 1, 7, 1, 300)])      # G = 12, pages that straddle 16-key blocks
def test_all_rows(norm, D, Hq, Hkv, bs, lo, hi):
    cfg = W.PagedDecode(f"dec_{D}", 5, Hq, Hkv, D, "bf16", bs, lo, hi, 1.0 / math.sqrt(D),
                        seed=77 + D)
    x, out, st = _run(cfg, norm)
    assert np.isfinite(out).all()  # the NaN page tails were never read
    rows = [(b, h, 0) for b in range(cfg.B) for h in range(Hq)]
    check_rows(out, st, rows, x.q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling,
               paged=_paged(x), where=f"decode D{D} G{Hq // Hkv} bs{bs}")


@pytest.mark.parametrize("norm", NORMS)
def test_window_and_softcap(norm):
    cfg = W.PagedDecode("dec_wc", 4, 8, 2, 128, "bf16", 16, 100, 2000, 1.0 / math.sqrt(128),
                        seed=91)
    x = W.make_paged(cfg)
    for window, cap in ((700, 0.0), (0, 5.0), (300, 20.0)):
        _, out, st = _run(cfg, norm, window, cap, x)
        rows = [(b, h, 0) for b in range(cfg.B) for h in range(cfg.Hq)]
        check_rows(out, st, rows, x.q, x.k_cache, x.v_cache, norm, True, window, cap,
                   cfg.scaling, paged=_paged(x), where=f"decode w{window} cap{cap}")


@pytest.mark.parametrize("norm", NORMS)
def test_block_table_permutation_invariance(norm):
    cfg = W.PagedDecode("dec_perm", 3, 8, 2, 128, "bf16", 16, 200, 1200, 0.09, seed=5)
    x = W.make_paged(cfg, nan_tail=False)
    _, a_out, a_st = _run(cfg, norm, x=x)
    # move every page to a new physical slot and rewrite the table accordingly
    nb = x.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb)
    k2 = x.k_cache[perm]
    v2 = x.v_cache[perm]
    t2 = x.block_table.clone()
    m = t2 >= 0
    t2[m] = inv[t2[m].long()].to(torch.int32)
    y = W.PagedInputs(x.q, k2, v2, t2, x.seq_lens, x.block_size, x.max_blocks)
    _, b_out, b_st = _run(cfg, norm, x=y)
    assert np.array_equal(a_out, b_out) and np.array_equal(a_st, b_st)


def test_zero_length_sequence():
    cfg = W.PagedDecode("dec_zero", 3, 8, 2, 128, "bf16", 16, 1, 100, 0.09, seed=9)
    x = W.make_paged(cfg)
    x.seq_lens[1] = 0
    for norm, want in (("softmax", (-math.inf, 0)), ("softmax1", (0, 1)),
                       ("sparsemax", (math.inf, 0)), ("entmax15", (math.inf, 0))):
        _, out, st = _run(cfg, norm, x=x)
        assert (out[1] == 0).all()
        assert (st[1, :, 0, 0] == want[0]).all() and (st[1, :, 0, 1] == want[1]).all()
        rows = [(b, h, 0) for b in (0, 2) for h in range(cfg.Hq)]
        check_rows(out, st, rows, x.q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling,
                   paged=_paged(x), where="decode zero-length neighbour")


def test_workspace_is_required():
    cfg = W.PagedDecode("dec_ws", 2, 8, 2, 128, "bf16", 16, 10, 40, 0.09, seed=4)
    x = W.make_paged(cfg, device="cuda")
    n = apn.attn_fwd_workspace_bytes(x.q, x.k_cache, x.v_cache, normalizer="softmax",
                                     causal=True, paged=_paged(x))
    assert n > 0
    small = torch.empty(n - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(apn.AttnError) as ei:
        apn.attn_fwd(x.q, x.k_cache, x.v_cache, normalizer="softmax", causal=True,
                     paged=_paged(x), workspace=small)
    assert ei.value.status == apn.ATTN_E_WORKSPACE


@pytest.mark.parametrize("norm", NORMS)
def test_decode_workload_sampled_rows(norm):
    """The full decode workload: B=64, Hq=32, Hkv=8, D=128, 1024..32768 keys."""
    cfg = W.DECODE
    x = W.make_paged(cfg, device="cuda")
    out, st = gpu_fwd(x.q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling, paged=_paged(x))
    assert np.isfinite(out).all()
    lens = x.seq_lens.cpu().numpy()
    if norm in ("sparsemax", "entmax15"):
        k = st[:, :, 0, 1]
        assert (k >= 1).all() and (k <= lens[:, None]).all()
    rng = np.random.default_rng(0)
    bs = [int(np.argmax(lens)), int(np.argmin(lens))] + list(rng.choice(64, 3, replace=False))
    rows = [(b, h, 0) for b in bs for h in (0, 5, 31)]
    xc = W.PagedInputs(x.q.cpu(), x.k_cache, x.v_cache, x.block_table.cpu(), x.seq_lens.cpu(),
                       x.block_size, x.max_blocks)
    check_rows(out, st, rows, xc.q, _CpuPages(x.k_cache), _CpuPages(x.v_cache), norm, True, 0,
               0.0, cfg.scaling, paged={"block_table": xc.block_table, "seq_lens": xc.seq_lens},
               where="decode workload")


class _CpuPages:
    """Page-wise host view of a device cache: the oracle pulls only the pages it reads."""

    def __init__(self, t):
        self.t = t
        self.shape = t.shape

    def __getitem__(self, i):
        return self.t[i].cpu()


def test_deterministic_repeat():
    cfg = W.PagedDecode("dec_det", 4, 32, 8, 128, "bf16", 16, 500, 5000, 0.09, seed=12)
    x = W.make_paged(cfg)
    for norm in NORMS:
        _, a_out, a_st = _run(cfg, norm, x=x)
        _, b_out, b_st = _run(cfg, norm, x=x)
        assert np.array_equal(a_out, b_out) and np.array_equal(a_st, b_st), norm


@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
@pytest.mark.parametrize("bs", (16, 7))
def test_flat_rows_overflow_candidate_buffer(norm, bs):
    """Near-uniform scores over 5000..9000 keys: every key is a threshold
    candidate, more than the solver's LDS buffer holds, so the search runs on
    the split lists in global memory (both split kernels)."""
    cfg = W.PagedDecode("dec_flat", 2, 8, 2, 128, "bf16", bs, 5000, 9000, 1e-3, seed=31)
    x, out, st = _run(cfg, norm)
    rows = [(b, h, 0) for b in range(cfg.B) for h in range(cfg.Hq)]
    # |z| < 0.1 for every key (scores of N(0,1) rows times 1e-3), so all
    # 5000+ keys of a row lie within 1 of its max and are candidates
    check_rows(out, st, rows, x.q, x.k_cache, x.v_cache, norm, True, 0, 0.0, cfg.scaling,
               paged=_paged(x), where=f"decode flat bs{bs}")
