"""GPU parity of the packed variable-length forward (attn_fwd_varlen): every
request is checked row by row against the oracle on its own slice.  Request
lengths include 0 and 1 and queries fewer than keys (bottom-right causal per
request); bf16 head dims 64/128/256 run on the matrix-core kernels, f32 on the
per-row kernel."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
import workloads as W
from parity import check_rows

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")


def _run_and_check(cfg, norm, sinks=None):
    q, k, v, cq, ck = W.make_varlen(cfg)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full_like(qd, float("nan"))
    st = torch.full((cfg.Hq, q.shape[0], 2), float("nan"), dtype=torch.float32, device="cuda")
    sd = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device="cuda")
    apn.attn_fwd_varlen(qd, kd, vd, cq.cuda(), ck.cuda(), max(cfg.q_lens), out, st,
                        normalizer=norm, causal=cfg.causal, window=cfg.window,
                        softcap=cfg.softcap, scaling=cfg.scaling, sinks=sd)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    st = st.double().cpu().numpy()
    assert np.isfinite(out).all()
    for r in range(len(cfg.q_lens)):
        q0, q1, k0, k1 = int(cq[r]), int(cq[r + 1]), int(ck[r]), int(ck[r + 1])
        if q1 == q0:
            continue
        view = lambda t, a, b: t[a:b].permute(1, 0, 2).unsqueeze(0)
        og = np.transpose(out[q0:q1], (1, 0, 2))[None]
        sg = st[:, q0:q1][None]
        rows = [(0, h, i) for h in range(cfg.Hq) for i in range(q1 - q0)]
        check_rows(og, sg, rows, view(q, q0, q1), view(k, k0, k1), view(v, k0, k1), norm,
                   cfg.causal, cfg.window, cfg.softcap, cfg.scaling,
                   where=f"varlen {cfg.name} request {r}", sinks=sinks)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D,causal,window,cap", [
    (64, True, 0, 0.0), (128, True, 40, 0.0), (256, True, 0, 20.0), (64, False, 0, 0.0)])
def test_varlen_bf16(norm, D, causal, window, cap):
    cfg = W.Varlen(f"vl{D}", (70, 0, 1, 129, 33, 200), (70, 5, 17, 300, 33, 260), 4, 2, D,
                   "bf16", causal, window, cap, 1.0 / math.sqrt(D), seed=400 + D)
    _run_and_check(cfg, norm)


@pytest.mark.parametrize("norm", NORMS)
def test_varlen_f32_per_row_kernel(norm):
    cfg = W.Varlen("vl_f32", (9, 1, 0, 20), (12, 3, 4, 20), 4, 1, 40, "f32", True, 0, 0.0, 0.2,
                   seed=411)
    _run_and_check(cfg, norm)


def test_varlen_softmax1_sinks():
    cfg = W.Varlen("vl_sink", (50, 90), (80, 90), 4, 2, 64, "bf16", True, 0, 0.0, 0.125, seed=413)
    _run_and_check(cfg, "softmax1", sinks=[-2.0, 0.5, 3.0, 0.0])


def test_varlen_matches_batched_call():
    # equal-length requests: the packed call equals the ordinary batched one
    cfg = W.Prefill("vl_eq", 3, 4, 2, 96, 96, 128, "bf16", True, 0, 0.0, 1 / math.sqrt(128),
                    seed=415)
    q, k, v = [x.cuda() for x in W.make_prefill(cfg)]
    ref, _ = apn.attn_fwd(q, k, v, normalizer="entmax15", causal=True, scaling=cfg.scaling)
    pack = lambda t: t.permute(0, 2, 1, 3).reshape(-1, t.shape[1], t.shape[3]).contiguous()
    cu = torch.arange(0, 4 * 96, 96, dtype=torch.int32, device="cuda")
    out, _ = apn.attn_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, 96, normalizer="entmax15",
                                 causal=True, scaling=cfg.scaling)
    torch.cuda.synchronize()
    assert torch.equal(out, pack(ref))
