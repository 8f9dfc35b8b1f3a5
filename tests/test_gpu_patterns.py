"""Support and mask patterns of every GPU path against the oracle, read by
one-hot value probes over every key (tests/patterns.py), on every row:
  * prefill at head dim 256, through softcap (with many keys near tau) and
    through CSR block masks (matrix-core and per-row kernels);
  * paged decode (split kernels of both page layouts, window, softcap) and
    chunked prefill over a paged cache;
  * rows whose support outgrows the prefill candidate buffers (extra
    passes), and decode rows whose support edge sits at a split floor.
The pages fix exact zeros off the support ("HF Attention Normalizers",
"Supported Normalizers"); keys within 1e-6 of tau may land either way."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from patterns import (gpu_pattern_paged, gpu_pattern_prefill, paged_rows_check, run_jobs,
                      slice_jobs)

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _rand(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def _f32(x):
    return x.float().numpy()


def check_prefill(q, k, v, norm, causal, window, softcap, scaling, where, block_mask=None):
    """Every row and every key of a contiguous forward against the oracle."""
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    bm_dev = None
    if block_mask is not None:
        num, idx, bq, bk = block_mask
        bm_dev = (torch.from_numpy(num).cuda(), torch.from_numpy(idx).cuda(), bq, bk)
    st = torch.full((*q.shape[:3], 2), float("nan"), device="cuda")
    out = torch.empty_like(qd)

    def run(vv, stats=None):
        apn.attn_fwd(qd, kd, vv, out, stats, normalizer=norm, causal=causal, window=window,
                     softcap=softcap, scaling=scaling, block_mask=bm_dev)
        return out

    run(vd, st)
    torch.cuda.synchronize()
    out_g = out.float().cpu().numpy()
    st_g = st.cpu().numpy()
    pat = gpu_pattern_prefill(kd, run)
    B, Hq = q.shape[:2]
    G = Hq // k.shape[1]
    bh = [(b, h) for b in range(B) for h in range(Hq)]
    jobs = slice_jobs(_f32(q), _f32(k), _f32(v), out_g, st_g, {x: pat[x] for x in bh}, norm,
                      causal, window, softcap, scaling,
                      "f32" if q.dtype == torch.float32 else "bf16", bh, G,
                      block_mask=block_mask, where=where)
    worst, nrows, fails = run_jobs(jobs)
    assert nrows == B * Hq * q.shape[2]
    assert not fails, "\n".join(fails)
    return worst, st_g


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("lq,lk,window,cap", [(300, 300, 0, 0.0), (260, 333, 100, 0.0),
                                               (129, 200, 64, 50.0)],
                         ids=["causal", "window100", "window64_cap50"])
def test_head_dim_256(norm, lq, lk, window, cap):
    q = _rand((1, 4, lq, 256), 700, 1.5)
    k = _rand((1, 2, lk, 256), 701, 1.5)
    v = _rand((1, 2, lk, 256), 702)
    check_prefill(q, k, v, norm, True, window, cap, 1.0 / 16.0, f"D256 w{window} cap{cap}")


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,sigma,cap", [(64, 1.5, 30.0), (128, 0.5, 50.0), (128, 2.0, 50.0),
                                         (256, 0.7, 50.0)])
def test_softcap(norm, D, sigma, cap):
    # small scores under a large cap: tanh near 0, where its evaluation must
    # stay accurate relative to its value; sigma 0.5 gives broad supports
    # with many keys close to tau
    q = _rand((1, 4, 290, D), 710 + D, sigma)
    k = _rand((1, 2, 290, D), 711 + D, sigma)
    v = _rand((1, 2, 290, D), 712 + D)
    check_prefill(q, k, v, norm, True, 0, cap, 1.0 / math.sqrt(D), f"softcap D{D} s{sigma}")


def _lists(rng, B, Hm, nqb, nkb, p):
    num = np.zeros((B, Hm, nqb), dtype=np.int32)
    idx = np.full((B, Hm, nqb, nkb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hm):
            for r in range(nqb):
                c = np.nonzero(rng.random(nkb) < p)[0]
                num[b, h, r] = len(c)
                idx[b, h, r, :len(c)] = c
    num[0, 0, nqb // 2] = 0
    return num, idx


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,bq,bk,causal,dtype", [(64, 128, 128, True, torch.bfloat16),
                                                  (256, 128, 64, False, torch.bfloat16),
                                                  (48, 16, 24, True, torch.float32)],
                         ids=["mfma_d64", "mfma_d256", "per_row_f32"])
def test_block_mask(norm, D, bq, bk, causal, dtype):
    rng = np.random.default_rng(D + bk)
    B, Hq, Hkv, Lq, Lk = 1, 4, 2, 400, 460
    q = _rand((B, Hq, Lq, D), 720 + D, 1.0, dtype)
    k = _rand((B, Hkv, Lk, D), 721 + D, 1.0, dtype)
    v = _rand((B, Hkv, Lk, D), 722 + D, 1.0, dtype)
    num, idx = _lists(rng, B, Hq, math.ceil(Lq / bq), math.ceil(Lk / bk), 0.5)
    check_prefill(q, k, v, norm, causal, 0, 0.0, 1.0 / math.sqrt(D), f"block mask D{D}",
                  block_mask=(num, idx, bq, bk))


@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
@pytest.mark.parametrize("D", [64, 128])
def test_support_beyond_candidate_buffers(norm, D):
    # flat scores (scaling 1e-4): every row's support holds nearly all of its
    # 445..700 keys, more than its two lanes' candidate buffers can hold
    # (at most 2 * 64 values per row at these head dims), so every long row
    # is finished by the extra passes over the key tiles
    q = _rand((1, 4, 256, D), 730 + D)
    k = _rand((1, 2, 700, D), 731 + D)
    v = _rand((1, 2, 700, D), 732 + D)
    _, st = check_prefill(q, k, v, norm, False, 0, 0.0, 1e-4, f"flat D{D}")
    assert (st[..., 1] > 2 * 64).all()  # provably beyond the buffers
    _, st = check_prefill(q, k, v, norm, True, 0, 0.0, 1e-4, f"flat causal D{D}")
    assert (st[..., 1] > 2 * 64).all()


def _paged(x):
    return {"block_table": x.block_table, "seq_lens": x.seq_lens, "block_size": x.block_size,
            "max_blocks": x.max_blocks}


def check_paged(cfg, x, q, norm, window, softcap, seqs, where):
    """Every row of the sequences `seqs` of a paged forward, pattern included."""
    qd = q.cuda()
    kc, vc = x.k_cache.cuda(), x.v_cache.cuda()
    table, lens = x.block_table.cuda(), x.seq_lens.cuda()
    paged = {"block_table": table, "seq_lens": lens, "block_size": x.block_size,
             "max_blocks": x.max_blocks}
    nbytes = apn.attn_fwd_workspace_bytes(qd, kc, vc, normalizer=norm, causal=True,
                                          window=window, softcap=softcap, scaling=cfg.scaling,
                                          paged=paged)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd)
    st = torch.full((*q.shape[:3], 2), float("nan"), device="cuda")

    def run(vv, stats=None):
        apn.attn_fwd(qd, kc, vv, out, stats, normalizer=norm, causal=True, window=window,
                     softcap=softcap, scaling=cfg.scaling, paged=paged, workspace=ws)
        return out

    run(vc, st)
    torch.cuda.synchronize()
    out_g = out.float().cpu().numpy()
    st_g = st.cpu().numpy()
    assert np.isfinite(out_g[seqs]).all()
    tab = x.block_table.cpu().numpy()
    ln = x.seq_lens.cpu().numpy()
    pats = gpu_pattern_paged(vc.clone(), tab, ln, seqs, q.shape[-1], run)
    rows = [(b, h, i) for b in seqs for h in range(q.shape[1]) for i in range(q.shape[2])]
    worst, fails = paged_rows_check(out_g, st_g, pats, q, x.k_cache.cpu(), x.v_cache.cpu(), tab,
                                    ln, rows, norm, window, softcap, cfg.scaling, "bf16", where)
    assert not fails, "\n".join(fails[:20])
    return st_g


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,Hq,Hkv,bs,lo,hi,window,cap", [
    (128, 32, 8, 16, 1, 1500, 0, 0.0),   # the decode workload's head layout
    (64, 8, 8, 16, 600, 1100, 300, 0.0),  # G = 1, several splits, window
    (256, 16, 2, 32, 30, 700, 0, 30.0),  # G = 8, larger pages, softcap
    (128, 12, 1, 7, 1, 300, 0, 0.0)])     # G = 12, pages that straddle 16-key blocks
def test_decode(norm, D, Hq, Hkv, bs, lo, hi, window, cap):
    cfg = W.PagedDecode(f"pdec_{D}", 4, Hq, Hkv, D, "bf16", bs, lo, hi, 1.0 / math.sqrt(D),
                        seed=740 + D + bs)
    x = W.make_paged(cfg)
    check_paged(cfg, x, x.q, norm, window, cap, list(range(cfg.B)), f"decode D{D} bs{bs}")


@pytest.mark.parametrize("norm", NORMS)
def test_chunked_prefill(norm):
    cfg = W.PagedDecode("pchunk_pat", 3, 4, 2, 64, "bf16", 16, 40, 400, 0.125, seed=750)
    x = W.make_paged(cfg)
    q = _rand((cfg.B, cfg.Hq, 80, cfg.D), 751)
    check_paged(cfg, x, q, norm, 0, 0.0, list(range(cfg.B)), "chunked prefill")


@pytest.mark.parametrize("norm", ("sparsemax", "entmax15"))
def test_decode_support_edge_at_split_floor(norm):
    """Rows whose whole support lies in one split of 512 keys: that split's
    floor steps reach the row's own threshold, so the largest split floor
    sits just below tau, next to the support's smallest members (for the
    first query head of each group, whose query direction the keys copy)."""
    D, Hq, Hkv = 128, 8, 2
    G = Hq // Hkv
    cfg = W.PagedDecode("pdec_edge", 4, Hq, Hkv, D, "bf16", 16, 1500, 2600, 1.0 / math.sqrt(D),
                        seed=760)
    x = W.make_paged(cfg, nan_tail=False)
    g = torch.Generator().manual_seed(761)
    bs = x.block_size
    for b in range(cfg.B):
        n = int(x.seq_lens[b])
        s = int(torch.randint(0, n // 512, (1,), generator=g))  # the split holding the support
        j = torch.arange(n)
        pages, slots = x.block_table[b, j // bs].long(), j % bs
        inside = (j >= s * 512) & (j < (s + 1) * 512)
        # split s: graded copies of the query direction; elsewhere weaker ones
        w = torch.where(inside, 0.9 + 0.2 * torch.rand(n, generator=g), torch.full((n,), 0.8))
        for kvh in range(Hkv):
            qv = x.q[b, kvh * G, 0].float()
            kk = w[:, None] * (4.0 * qv / qv.norm())[None] + 0.15 * torch.randn(n, D, generator=g)
            x.k_cache[pages, slots, kvh] = kk.to(torch.bfloat16)
    st = check_paged(cfg, x, x.q, norm, 0, 0.0, list(range(cfg.B)), "decode edge")
    assert (st[:, ::G, 0, 1] >= 2).all()
