"""Weight patterns of the GPU path, read through one-hot value probes, and
every-row comparisons against the oracle.

A probe run keeps q and k and replaces V by unit vectors: the value row of
key j0 + c is e_c for c < D (every kv head), all other value rows are zero.
Then out[..., c] is the weight of key j0 + c itself, and exact zeros stay
exact zeros through the products, so out[..., c] > 0 exactly when that key
has a nonzero weight.  Scores, mask and threshold do not depend on V, so the
probe runs see the weights of the regular run; Lk / D runs cover every key.

The oracle side runs in worker processes (``spawn``: they never touch the
GPU) over (batch, head) slices cut into row chunks, each compared row by row:
  * out max-abs error against the bf16 / f32 bar,
  * row statistics (``parity.compare_stats``),
  * the pattern: a key is nonzero on the GPU exactly when it is in the
    oracle's support (softmax family: exactly the allowed keys), except keys
    whose z lies within 1e-6 of the oracle's tau (the exclusion band).
"""

import concurrent.futures
import multiprocessing
import os

import numpy as np

from oracle import attention_forward, paged_attention_forward

BAND = 1e-6
TOL_OUT = {"bf16": 2e-2, "f32": 1e-5}


def workers():
    return max(1, min(16, os.cpu_count() or 1))


_POOL = None
_ONE_THREAD = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _worker_init():
    # one BLAS thread per worker: the workers already use every core
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def pool():
    """One pool of spawned worker processes for the whole test session, each
    limited to one BLAS thread (spawned children read these variables at
    start-up; the parent's own settings are restored)."""
    global _POOL
    if _POOL is None:
        saved = {k: os.environ.get(k) for k in _ONE_THREAD}
        os.environ.update({k: "1" for k in _ONE_THREAD})
        try:
            _POOL = concurrent.futures.ProcessPoolExecutor(
                max_workers=workers(), mp_context=multiprocessing.get_context("spawn"),
                initializer=_worker_init)
            _POOL.submit(int).result()  # start the workers while the variables hold
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    return _POOL


# --------------------------------------------------------------------------
# GPU side (torch and the library are imported here only)

def gpu_pattern_prefill(kd, run, bh=None):
    """Pattern of a contiguous-K/V forward, [B, Hq, Lq, Lk] bool (or [Lq, Lk]
    for the single (b, h) slice ``bh``).  ``run(v)`` launches the forward with
    value tensor v (shape and dtype of kd) and returns its output tensor."""
    import torch
    B, Hkv, Lk, D = kd.shape
    v = torch.zeros_like(kd)
    eye = torch.eye(D, dtype=kd.dtype, device=kd.device)
    pat = None
    for j0 in range(0, Lk, D):
        n = min(D, Lk - j0)
        v.zero_()
        v[:, :, j0:j0 + n, :] = eye[:n]
        out = run(v)
        torch.cuda.synchronize()
        o = out[bh[0], bh[1]] if bh is not None else out
        g = (o[..., :n] > 0).cpu().numpy()
        if pat is None:
            pat = np.zeros((*g.shape[:-1], Lk), dtype=bool)
        pat[..., j0:j0 + n] = g
    v.zero_()
    return pat


def gpu_pattern_paged(v_cache, table, lens, seqs, D, run):
    """Patterns of a paged forward for the sequences ``seqs``: {b: bool [Hq,
    Lq, lens[b]]}.  ``v_cache`` is the device value cache (overwritten: every
    live slot is set to zero and the probes written into it; slots past a
    sequence's end keep their contents); table / lens are host arrays."""
    import torch
    bs = v_cache.shape[1]
    live = ~torch.isnan(v_cache)
    v_cache.masked_fill_(live, 0.0)
    maxlen = max(int(lens[b]) for b in seqs)
    pats = {}
    for j0 in range(0, maxlen, D):
        pg, sl, col, spans = [], [], [], []
        for b in seqs:
            n = min(D, int(lens[b]) - j0)
            if n <= 0:
                continue
            j = np.arange(j0, j0 + n)
            pg.append(np.asarray(table[b])[j // bs])
            sl.append(j % bs)
            col.append(np.arange(n))
            spans.append((b, n))
        P = torch.from_numpy(np.concatenate(pg).astype(np.int64)).to(v_cache.device)
        S = torch.from_numpy(np.concatenate(sl).astype(np.int64)).to(v_cache.device)
        C = torch.from_numpy(np.concatenate(col).astype(np.int64)).to(v_cache.device)
        v_cache[P, S, :, C] = 1.0
        out = run(v_cache)
        torch.cuda.synchronize()
        o = out.cpu()
        for b, n in spans:
            g = (o[b, :, :, :n] > 0).numpy()
            if b not in pats:
                pats[b] = np.zeros((*g.shape[:-1], int(lens[b])), dtype=bool)
            pats[b][..., j0:j0 + n] = g
        v_cache[P, S, :, C] = 0.0
    return pats


# --------------------------------------------------------------------------
# oracle side

def _row_check(norm, dtype, out_g, st_g, pat_g, out_o, st_o, det, where):
    """Failures (strings) of one row; returns (max-abs error, failures)."""
    from parity import compare_stats
    idx, p, z = det
    err = float(np.abs(out_g - out_o).max()) if out_g.size else 0.0
    fails = []
    if not err <= TOL_OUT[dtype]:
        fails.append(f"{where}: out max-abs {err:.3e}")
    sparse = norm in ("sparsemax", "entmax15")
    tau = float(st_o[0])
    band = 0
    if sparse and np.isfinite(tau) and len(z):
        band = int(np.sum(np.abs(np.asarray(z) - tau) <= BAND))
    try:
        compare_stats(st_g, st_o, norm, len(idx), band, where=where)
    except AssertionError as e:
        fails.append(str(e))
    if pat_g is not None:
        want = np.zeros(pat_g.shape[-1], dtype=bool)
        want[np.asarray(idx)[np.asarray(p) > 0]] = True
        mism = pat_g != want
        if sparse and len(idx) and np.isfinite(tau):
            inband = np.zeros_like(mism)
            inband[np.asarray(idx)] = np.abs(np.asarray(z) - tau) <= BAND
            mism &= ~inband
        if mism.any():
            fails.append(f"{where}: {int(mism.sum())} pattern mismatches "
                         f"(keys {np.nonzero(mism)[0][:8].tolist()})")
    return err, fails


def slice_job(job):
    """Oracle check of query rows ``rows`` of one (batch, head) slice.

    job: dict with q [Lq, D], k, v [Lk, D] (float32 arrays holding the exact
    input values), norm, causal, window, softcap, scaling, dtype ("bf16" /
    "f32"), rows (query indices), out_g [len(rows), D], st_g [len(rows), 2],
    pat_g (packed bits [len(rows), ceil(Lk / 8)] or None), block_mask (the
    slice's (num [1,1,nqb], idx [1,1,nqb,m], bq, bk) or None), where.
    Returns (max-abs error, number of rows checked, failures[:20]).
    """
    q, k, v = job["q"][None, None], job["k"][None, None], job["v"][None, None]
    rows = [(0, 0, int(i)) for i in job["rows"]]
    out_o, st_o, det = attention_forward(q, k, v, job["norm"], job["causal"], job["window"],
                                         job["softcap"], job["scaling"], rows=rows,
                                         return_probs=True, block_mask=job.get("block_mask"))
    Lk = k.shape[2]
    pat = None
    if job.get("pat_g") is not None:
        pat = np.unpackbits(job["pat_g"], axis=-1, count=Lk).astype(bool)
    worst, fails = 0.0, []
    for r, (_, _, i) in enumerate(rows):
        e, f = _row_check(job["norm"], job["dtype"], job["out_g"][r], job["st_g"][r],
                          None if pat is None else pat[r], out_o[r], st_o[r], det[r],
                          f"{job['where']} row {i}")
        worst = max(worst, e)
        fails += f
    return worst, len(rows), fails[:20]


def slice_jobs(q, k, v, out_g, st_g, pat_g, norm, causal, window, softcap, scaling, dtype,
               bh_list, G, chunk=1024, block_mask=None, where=""):
    """Jobs for the (b, h) slices in bh_list, cut into row chunks.  q, k, v
    are float32 arrays [B, H, L, D]; out_g, st_g the GPU results [B, Hq, Lq,
    ...]; pat_g a dict (b, h) -> bool [Lq, Lk] or None."""
    jobs = []
    Lq = q.shape[2]
    for b, h in bh_list:
        kvh = h // G
        pat = None if pat_g is None else np.packbits(pat_g[(b, h)], axis=-1)
        bm = None
        if block_mask is not None:
            num, idx, bq, bk = block_mask
            hm = 0 if num.shape[1] == 1 else h
            bm = (num[b:b + 1, hm:hm + 1], idx[b:b + 1, hm:hm + 1], bq, bk)
        for i0 in range(0, Lq, chunk):
            i1 = min(Lq, i0 + chunk)
            jobs.append(dict(q=q[b, h], k=k[b, kvh], v=v[b, kvh], norm=norm, causal=causal,
                             window=window, softcap=softcap, scaling=scaling, dtype=dtype,
                             rows=np.arange(i0, i1), out_g=out_g[b, h, i0:i1],
                             st_g=st_g[b, h, i0:i1],
                             pat_g=None if pat is None else pat[i0:i1], block_mask=bm,
                             where=f"{where} {norm} (b={b}, h={h})"))
    return jobs


def run_jobs(jobs):
    """Runs the jobs in worker processes; returns (max error, rows, failures)."""
    worst, nrows, fails = 0.0, 0, []
    for e, n, f in pool().map(slice_job, jobs):
        worst = max(worst, e)
        nrows += n
        fails += f
    return worst, nrows, fails


def paged_rows_check(out_g, st_g, pats, q, k_cache, v_cache, table, lens, rows, norm, window,
                     softcap, scaling, dtype, where=""):
    """Every listed row of a paged forward against the oracle (in this
    process): out, stats and, with ``pats`` ({b: [Hq, Lq, n]}), the pattern."""
    out_o, st_o, det = paged_attention_forward(q, k_cache, v_cache, table, lens, norm, True,
                                               window, softcap, scaling, rows=rows,
                                               return_probs=True)
    worst, fails = 0.0, []
    for r, (b, h, i) in enumerate(rows):
        pat = None if pats is None else pats[b][h, i]
        e, f = _row_check(norm, dtype, out_g[b, h, i], st_g[b, h, i], pat, out_o[r], st_o[r],
                          det[r], f"{where} {norm} row {(b, h, i)}")
        worst = max(worst, e)
        fails += f
    return worst, fails
