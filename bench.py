"""Throughput of the attention forward with pluggable normalizers on one MI355X.

One step = one forward of the Llama-3.2-1B-shaped prefill workload (B=4,
Hq=32, Hkv=8, L=2048, head dim 64, bf16, causal, scaling 1/8) for each of the
four normalizers (softmax, softmax1, sparsemax, 1.5-entmax) on the same
synthetic inputs, already resident in HBM.  The metric is credited TFLOP/s:
4 * head_dim FLOPs per unmasked (query, key) pair, the same for every
normalizer (recomputed score passes of the sparse normalizers are not
credited).  `value` is the whole step (4 launches) over the wall clock of the
timed steps.

Also reported (not part of `value`): per-launch medians over the timed steps
(HIP events on the launch stream), the roofline of the slowest kernel, the
Qwen3-1.7B-shaped prefill at three score scales (mean support size per scale),
the Gemma-2-9B-shaped local layer, the paged-decode workload in GB/s (skip
with --no-decode) and the fp64 CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode]
       [--no-extra] [--no-cpu-baseline]
       python bench.py --kernel WORKLOAD:NORMALIZER [--steps K] [--warmup W]
Prints one JSON line.  --kernel launches one kernel configuration only (for
profiler runs): WORKLOAD is one of llama, qwen0.5, qwen1, qwen2, gemma,
decode, chunk (chunked prefill over the decode cache, 512 queries per
sequence).
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources of the prefill kernels and the build script that sets their
# compiler flags (the counter summary is tied to their hash)
_BUILD_PY = os.path.join(ROOT, "attention_pluggable_normalizers_amd", "build.py")
PREFILL_SRCS = [os.path.join(ROOT, "attention_pluggable_normalizers_amd", "csrc", f)
                for f in ("prefill.hip", "tiles.h", "common.h")] + [_BUILD_PY]
DECODE_SRCS = [os.path.join(ROOT, "attention_pluggable_normalizers_amd", "csrc", f)
               for f in ("decode.hip", "common.h")] + [_BUILD_PY]


def credited_pairs(cfg):
    """Unmasked (query, key) pairs of a prefill workload (integer count)."""
    total = 0
    for i in range(cfg.Lq):
        qp = i + cfg.Lk - cfg.Lq
        hi = max(0, min(cfg.Lk, qp + 1) if cfg.causal else cfg.Lk)
        lo = min(max(0, qp - cfg.window + 1) if cfg.window else 0, hi)
        total += hi - lo
    return total * cfg.B * cfg.Hq


def decode_bytes(x, cfg, seq_lens, norm, support=None):
    """Bytes the paged decode must move for one normalizer.

    softmax / softmax1: every live K and V row.  sparsemax / entmax15: every
    live K row (all scores are needed for the threshold) but only the V rows
    of the support; `support` is the per-(sequence, query head) support size
    from row_stats, so V is counted once per query head (an upper bound on
    the union over the heads of a group).  Plus q, out, the used block-table
    entries and the sequence lengths.
    """
    live = int(sum(seq_lens))
    k = live * cfg.Hkv * cfg.D * 2
    if norm in ("softmax", "softmax1"):
        v = k
    else:
        v = int(round(float(support.sum()))) * cfg.D * 2
    q = cfg.B * cfg.Hq * cfg.D * 2
    table = sum(x.extra["pages"]) * 4
    return k + v + q + q + table + cfg.B * 4


def median_us(pairs):
    ts = sorted(a.elapsed_time(b) for a, b in pairs)
    return ts[len(ts) // 2] * 1e3


def time_launches(f, reps, warmup):
    """Median launch time (us) with HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return median_us(evs)


def traffic_for(kernel_key, family="prefill"):
    """HBM bytes per launch (all kernels of the call) from the committed
    counter summary, or None when the family's kernel sources changed since
    the counters were taken."""
    srcs = PREFILL_SRCS if family == "prefill" else DECODE_SRCS
    try:
        rec = json.load(open(TRAFFIC_FILE))
        src = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get(f"{family}_src_sha256") != src or kernel_key not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel_key]
    return int(k["read_bytes"] + k["write_bytes"])


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), else the platform's."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine() or "host"


def cpu_baseline(cfg, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same workload (host cores)."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import attention_forward

    q, k, v = (x.double().numpy() for x in W.make_prefill(cfg))  # exact upcast, untimed
    threads = torch.get_num_threads()
    # sample: query rows spread over the sequence of one (batch, head) pair,
    # every normalizer, until the time budget is spent
    rng = np.random.default_rng(0)
    rows_done = 0
    flops = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        i = int(rng.integers(cfg.Lq))
        b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq))
        for norm in cfg.normalizers:
            attention_forward(q, k, v, norm, cfg.causal, cfg.window, cfg.softcap, cfg.scaling,
                              rows=[(b, h, i)])
        n = min(cfg.Lk, i + cfg.Lk - cfg.Lq + 1) if cfg.causal else cfg.Lk
        flops += 4 * cfg.D * n * len(cfg.normalizers)
        rows_done += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} query rows x {len(cfg.normalizers)} normalizers of {cfg.name} "
                      f"(fp64 NumPy oracle, one row per call), {dt:.1f} s",
            "cpu": cpu_model(), "logical_cpus": os.cpu_count()}


def extra_prefill(apn, W, dev, reps=10):
    """Qwen3-1.7B-shaped sweep over the score scale, and the Gemma-2-9B-shaped
    local layer: median launch time, credited TFLOP/s, mean support size."""
    import torch
    res = {}
    for cfg in (W.qwen(0.5), W.qwen(1.0), W.qwen(2.0), W.GEMMA):
        q, k, v = [x.to(dev) for x in W.make_prefill(cfg)]
        out = torch.empty_like(q)
        st = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=dev)
        flops = 4 * cfg.D * credited_pairs(cfg)
        per = {}
        for n in cfg.normalizers:
            f = lambda: apn.attn_fwd(q, k, v, out, st, normalizer=n, causal=cfg.causal,
                                     window=cfg.window, softcap=cfg.softcap, scaling=cfg.scaling)
            us = time_launches(f, reps, 2)
            per[n] = {"us": round(us, 1), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                      "pct_bf16_peak": round(100 * flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2)}
            if n in ("sparsemax", "entmax15"):
                per[n]["mean_support"] = round(float(st[..., 1].mean()), 2)
        res[cfg.name] = {"B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "L": cfg.Lq, "head_dim": cfg.D,
                         "window": cfg.window, "softcap": cfg.softcap,
                         "credited_flop_per_launch": flops, "per_normalizer": per}
        del q, k, v, out, st
        torch.cuda.empty_cache()
    return res


def largest_roofline(W, workloads):
    """Roofline of the slowest kernel of the largest workload (the
    Qwen3-1.7B-shaped sweep: 2 x 16 heads x 8192 x 8192 keys, every score
    scale), from the launch times measured in extra_prefill."""
    best = None
    for cfg in (W.qwen(0.5), W.qwen(1.0), W.qwen(2.0)):
        rec = workloads[cfg.name]
        for n, r in rec["per_normalizer"].items():
            if best is None or r["us"] > best[2]:
                best = (cfg, n, r["us"], rec["credited_flop_per_launch"])
    cfg, n, us, flops = best
    achieved = flops / (us * 1e-6) / 1e12
    return {"kernel": f"prefill {n} ({cfg.name})", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(f"{cfg.name}:{n}")}


def backward_bench(apn, cfg, q, k, v, norms, pairs, reps=20):
    """Backward (attn_bwd) of the same workload from the forward's row
    statistics and output: median time and TFLOP/s on the conventional
    10 * D * pairs (the five products of the backward: scores, dP, dV, dQ, dK)."""
    import torch
    g = torch.Generator(device=q.device).manual_seed(cfg.seed + 17)
    do = torch.randn(q.shape, generator=g, device=q.device).to(q.dtype)
    st = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    flops = 10 * cfg.D * pairs
    per = {}
    for n in norms:
        out, _ = apn.attn_fwd(q, k, v, None, st, normalizer=n, causal=cfg.causal,
                              scaling=cfg.scaling)
        f = lambda: apn.attn_bwd(q, k, v, do, st, normalizer=n, causal=cfg.causal,
                                 scaling=cfg.scaling, dq=dq, dk=dk, dv=dv, out=out)
        us = time_launches(f, reps, 3)
        per[n] = {"us": round(us, 1), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 2)}
    return {"workload": cfg.name, "credited_flop_per_launch": flops, "per_normalizer": per}


def decode_bench(apn, W, dev, reps, chunk=0):
    import torch
    dcfg = W.DECODE
    x = W.make_paged(dcfg, device=dev)
    lens = x.seq_lens.cpu().tolist()
    paged = {"block_table": x.block_table, "seq_lens": x.seq_lens,
             "block_size": x.block_size, "max_blocks": x.max_blocks}
    dout = torch.empty_like(x.q)
    dst = torch.empty(*x.q.shape[:3], 2, dtype=torch.float32, device=dev)
    dres = {}
    for n in dcfg.normalizers:
        ws_n = apn.attn_fwd_workspace_bytes(x.q, x.k_cache, x.v_cache, normalizer=n,
                                            causal=True, scaling=dcfg.scaling, paged=paged)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        f = lambda: apn.attn_fwd(x.q, x.k_cache, x.v_cache, dout, dst, normalizer=n,
                                 causal=True, scaling=dcfg.scaling, paged=paged, workspace=ws)
        us = time_launches(f, reps, 3)
        nbytes = decode_bytes(x, dcfg, lens, n, dst[..., 1].cpu())
        dres[n] = {"us": round(us, 1), "bytes": nbytes,
                   "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del ws
    dom = max(dres, key=lambda n: dres[n]["us"])
    res = {"workload": dcfg.name, "B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv,
           "head_dim": dcfg.D, "block_size": dcfg.block_size, "live_keys": int(sum(lens)),
           "per_normalizer": dres,
           "roofline": {"kernel": f"paged decode {dom}", "bound": "hbm",
                        "achieved": dres[dom]["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": dres[dom]["frac_hbm_peak"],
                        "traffic": traffic_for(f"{dcfg.name}:{dom}", "decode")}}
    if chunk:
        res["chunked_prefill"] = chunk_bench(apn, x, dcfg, lens, paged, dev, chunk)
    return res


def chunk_bench(apn, x, dcfg, lens, paged, dev, Lq, reps=5):
    """Chunked prefill over the decode workload's paged cache: the last Lq
    tokens of every sequence as queries (bottom-right causal against the
    sequence's own length), on the matrix-core kernels through the block
    table.  Credited FLOPs: 4 * D * unmasked pairs."""
    import torch
    g = torch.Generator(device=dev).manual_seed(dcfg.seed + 31)
    q = torch.randn(dcfg.B, dcfg.Hq, Lq, dcfg.D, generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    st = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=dev)
    pairs = sum(Lq * (n - Lq) + Lq * (Lq + 1) // 2 if n >= Lq else n * (n + 1) // 2 for n in lens)
    flops = 4 * dcfg.D * pairs * dcfg.Hq
    per = {}
    for n in dcfg.normalizers:
        f = lambda: apn.attn_fwd(q, x.k_cache, x.v_cache, out, st, normalizer=n, causal=True,
                                 scaling=dcfg.scaling, paged=paged)
        us = time_launches(f, reps, 2)
        per[n] = {"us": round(us, 1), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                  "pct_bf16_peak": round(100 * flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    del q, out, st
    torch.cuda.empty_cache()
    return {"Lq": Lq, "credited_flop_per_launch": flops, "per_normalizer": per}


KERNEL_WORKLOADS = ("llama", "qwen0.5", "qwen1", "qwen2", "gemma", "decode", "chunk")


def kernel_only(apn, W, dev, spec, steps, warmup):
    """Launch one workload / normalizer pair `warmup` + `steps` times (for
    profiler runs) and return its median launch time and credited rate."""
    import torch
    name, _, norm = spec.partition(":")
    if name not in KERNEL_WORKLOADS or norm not in W.NORMALIZERS:
        raise SystemExit(f"--kernel takes WORKLOAD:NORMALIZER with WORKLOAD in {KERNEL_WORKLOADS}"
                         f" and NORMALIZER in {W.NORMALIZERS}")
    res = {"kernel": spec, "steps": steps, "warmup": warmup}
    if name in ("decode", "chunk"):
        dcfg = W.DECODE
        x = W.make_paged(dcfg, device=dev)
        lens = x.seq_lens.cpu().tolist()
        paged = {"block_table": x.block_table, "seq_lens": x.seq_lens,
                 "block_size": x.block_size, "max_blocks": x.max_blocks}
        if name == "decode":
            q = x.q
            nbytes = apn.attn_fwd_workspace_bytes(q, x.k_cache, x.v_cache, normalizer=norm,
                                                  causal=True, scaling=dcfg.scaling, paged=paged)
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        else:
            g = torch.Generator(device=dev).manual_seed(dcfg.seed + 31)
            Lq = 512
            q = torch.randn(dcfg.B, dcfg.Hq, Lq, dcfg.D, generator=g, device=dev).to(torch.bfloat16)
            ws = None
            pairs = sum(Lq * (n - Lq) + Lq * (Lq + 1) // 2 if n >= Lq else n * (n + 1) // 2
                        for n in lens)
            res["credited_flop_per_launch"] = 4 * dcfg.D * pairs * dcfg.Hq
        out = torch.empty_like(q)
        st = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=dev)
        f = lambda: apn.attn_fwd(q, x.k_cache, x.v_cache, out, st, normalizer=norm, causal=True,
                                 scaling=dcfg.scaling, paged=paged, workspace=ws)
        us = time_launches(f, steps, warmup)
        if name == "decode":
            res["bytes_per_launch"] = decode_bytes(x, dcfg, lens, norm, st[..., 1].cpu())
            res["GB/s"] = round(res["bytes_per_launch"] / (us * 1e-6) / 1e9, 1)
    else:
        cfg = {"llama": W.LLAMA, "qwen0.5": W.qwen(0.5), "qwen1": W.qwen(1.0),
               "qwen2": W.qwen(2.0), "gemma": W.GEMMA}[name]
        q, k, v = [x.to(dev) for x in W.make_prefill(cfg)]
        out = torch.empty_like(q)
        st = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=dev)
        f = lambda: apn.attn_fwd(q, k, v, out, st, normalizer=norm, causal=cfg.causal,
                                 window=cfg.window, softcap=cfg.softcap, scaling=cfg.scaling)
        us = time_launches(f, steps, warmup)
        res["credited_flop_per_launch"] = 4 * cfg.D * credited_pairs(cfg)
    res["us"] = round(us, 1)
    if "credited_flop_per_launch" in res:
        tf = res["credited_flop_per_launch"] / (us * 1e-6) / 1e12
        res["TFLOP/s"] = round(tf, 1)
        res["pct_bf16_peak"] = round(100 * tf / PEAK_BF16_TFLOPS, 2)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(a reference for scaling hardware byte counters)")
    ap.add_argument("--kernel", default="",
                    help="WORKLOAD:NORMALIZER -- launch only this kernel configuration "
                         "(warmup + steps launches) and print its median time")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this forward has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_pluggable_normalizers_amd as apn
    import workloads as W

    apn.load_library()
    dev = torch.device("cuda:0")
    if args.kernel:
        print(json.dumps(kernel_only(apn, W, dev, args.kernel, args.steps, args.warmup)), flush=True)
        return
    cfg = W.LLAMA
    q, k, v = [x.to(dev) for x in W.make_prefill(cfg)]
    out = torch.empty_like(q)
    stats = torch.empty(*q.shape[:3], 2, dtype=torch.float32, device=dev)
    norms = list(cfg.normalizers)
    pairs = credited_pairs(cfg)
    flops_per_launch = 4 * cfg.D * pairs

    def launch(norm):
        apn.attn_fwd(q, k, v, out, stats, normalizer=norm, causal=cfg.causal, window=cfg.window,
                     softcap=cfg.softcap, scaling=cfg.scaling)

    for _ in range(args.warmup):
        for n in norms:
            launch(n)
    torch.cuda.synchronize()

    # timed region: K steps; each launch bracketed by events on the launch stream
    evs = {n: [] for n in norms}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for n in norms:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            launch(n)
            e1.record()
            evs[n].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_norm_us = {n: median_us(evs[n]) for n in norms}
    ms_per_step = wall * 1e3 / args.steps
    value = flops_per_launch * len(norms) / (ms_per_step * 1e-3) / 1e12

    dom = max(norms, key=lambda n: per_norm_us[n])
    achieved = flops_per_launch / (per_norm_us[dom] * 1e-6) / 1e12
    result = {
        "metric": "attention fwd TFLOP/s per normalizer + % bf16 MFMA peak; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "L": cfg.Lq,
                   "head_dim": cfg.D, "causal": cfg.causal, "scaling": cfg.scaling,
                   "normalizers": norms, "credited_pairs": pairs,
                   "credited_flop_per_launch": flops_per_launch, "parallelism": "single GPU"},
        "per_normalizer": {n: {"us": round(per_norm_us[n], 1),
                               "TFLOP/s": round(flops_per_launch / (per_norm_us[n] * 1e-6) / 1e12, 1),
                               "pct_bf16_peak": round(100 * flops_per_launch /
                                                      (per_norm_us[n] * 1e-6) / 1e12 /
                                                      PEAK_BF16_TFLOPS, 2)} for n in norms},
        "roofline": {"kernel": f"prefill {dom}", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(f"{cfg.name}:{dom}")},
    }

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n * 4
        del src, dst

    if not args.no_extra:
        result["backward"] = backward_bench(apn, cfg, q, k, v, norms, pairs)
    del q, k, v, out, stats
    torch.cuda.empty_cache()
    if not args.no_extra:
        result["prefill_workloads"] = extra_prefill(apn, W, dev)
        result["roofline_largest"] = largest_roofline(W, result["prefill_workloads"])
    if not args.no_decode:
        result["decode"] = decode_bench(apn, W, dev, max(3, args.steps),
                                        chunk=0 if args.no_extra else 512)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
