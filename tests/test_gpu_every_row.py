"""Every row of the full-size workloads against the oracle, in the launch
configuration bench.py times, with the support / mask pattern of every key
read by one-hot value probes (tests/patterns.py):
  * Llama-3.2-1B-shaped prefill: every row of every head, four normalizers;
  * Qwen3-1.7B-shaped prefill at each score scale: every row of one whole
    (batch, head) slice, sparsemax, 1.5-entmax and softmax1;
  * Gemma-2-9B-shaped local layer: every row of one whole slice;
  * paged decode workload: every head of eight complete sequences.
Out within the bf16 bar, row statistics as in tests/parity.py, patterns
bit-exact outside the 1e-6 band around tau."""

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from patterns import (gpu_pattern_paged, gpu_pattern_prefill, paged_rows_check, run_jobs,
                      slice_jobs)

pytestmark = pytest.mark.gpu


def _prefill_every_row(cfg, norm, bh_list):
    import time
    t0 = time.time()
    q, k, v = W.make_prefill(cfg)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    st = torch.full((*q.shape[:3], 2), float("nan"), device="cuda")

    def run(vv, stats=None):
        apn.attn_fwd(qd, kd, vv, out, stats, normalizer=norm, causal=cfg.causal,
                     window=cfg.window, softcap=cfg.softcap, scaling=cfg.scaling)
        return out

    run(vd, st)
    torch.cuda.synchronize()
    out_g = out.float().cpu().numpy()
    st_g = st.cpu().numpy()
    assert np.isfinite(out_g).all()
    pats = {}
    if len(bh_list) == cfg.B * cfg.Hq:
        full = gpu_pattern_prefill(kd, run)
        pats = {x: full[x] for x in bh_list}
    else:
        for x in bh_list:
            pats[x] = gpu_pattern_prefill(kd, run, bh=x)
    t1 = time.time()
    del qd, kd, vd, out
    torch.cuda.empty_cache()
    jobs = slice_jobs(q.float().numpy(), k.float().numpy(), v.float().numpy(), out_g, st_g, pats,
                      norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling, "bf16", bh_list,
                      cfg.Hq // cfg.Hkv, chunk=2048 if len(bh_list) > 16 else 512,
                      where=cfg.name)
    t2 = time.time()
    worst, nrows, fails = run_jobs(jobs)
    print(f"timing: gpu+inputs {t1 - t0:.1f} s, jobs {t2 - t1:.1f} s, oracle {time.time() - t2:.1f} s")
    assert nrows == len(bh_list) * cfg.Lq
    assert not fails, "\n".join(fails[:20])
    print(f"{cfg.name} {norm}: {nrows} rows, out max-abs {worst:.3e}")
    return st_g


@pytest.mark.parametrize("norm", W.NORMALIZERS)
def test_llama_every_row(norm):
    cfg = W.LLAMA
    _prefill_every_row(cfg, norm, [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)])


@pytest.mark.parametrize("sigma", W.QWEN_SIGMAS)
@pytest.mark.parametrize("norm", ("sparsemax", "entmax15", "softmax1"))
def test_qwen_whole_slice(norm, sigma):
    _prefill_every_row(W.qwen(sigma), norm, [(1, 13)])


@pytest.mark.parametrize("norm", ("softmax", "softmax1"))
def test_gemma_whole_slice(norm):
    _prefill_every_row(W.GEMMA, norm, [(0, 9)])


class _CpuPages:
    """Page-wise host view of a device cache: the oracle pulls only the pages it reads."""

    def __init__(self, t):
        self.t = t
        self.shape = t.shape

    def __getitem__(self, i):
        return self.t[i].cpu()


@pytest.mark.parametrize("norm", W.NORMALIZERS)
def test_decode_eight_sequences(norm):
    cfg = W.DECODE
    x = W.make_paged(cfg, device="cuda")
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens,
             "block_size": x.block_size, "max_blocks": x.max_blocks}
    nbytes = apn.attn_fwd_workspace_bytes(x.q, x.k_cache, x.v_cache, normalizer=norm,
                                          causal=True, scaling=cfg.scaling, paged=paged)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x.q)
    st = torch.full((*x.q.shape[:3], 2), float("nan"), device="cuda")

    def run(vv, stats=None):
        apn.attn_fwd(x.q, x.k_cache, vv, out, stats, normalizer=norm, causal=True,
                     scaling=cfg.scaling, paged=paged, workspace=ws)
        return out

    run(x.v_cache, st)
    torch.cuda.synchronize()
    out_g = out.float().cpu().numpy()
    st_g = st.cpu().numpy()
    assert np.isfinite(out_g).all()
    lens = x.seq_lens.cpu().numpy()
    tab = x.block_table.cpu().numpy()
    # the longest and shortest sequences and six more
    rng = np.random.default_rng(11)
    seqs = [int(np.argmax(lens)), int(np.argmin(lens))]
    seqs += [int(b) for b in rng.permutation(cfg.B) if int(b) not in seqs][:6]
    pats = gpu_pattern_paged(x.v_cache.clone(), tab, lens, seqs, cfg.D, run)
    rows = [(b, h, 0) for b in seqs for h in range(cfg.Hq)]
    worst, fails = paged_rows_check(out_g, st_g, pats, x.q.cpu(), _CpuPages(x.k_cache),
                                    _CpuPages(x.v_cache), tab, lens, rows, norm, 0, 0.0,
                                    cfg.scaling, "bf16", "decode workload")
    assert not fails, "\n".join(fails[:20])
    print(f"decode {norm}: {len(rows)} rows, out max-abs {worst:.3e}")
