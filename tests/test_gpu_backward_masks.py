"""GPU parity of the backward under block masks (attn_bwd with a block mask)
and over packed variable-length batches (attn_bwd_varlen), against the
float64 oracle, from the row statistics the GPU forward saved.  Both run on
the per-row kernels (f32 and bf16).

Block masks: several block shapes, one list shared by all heads or one per
head, a query block with an empty list, lists with ignored entries (out of
range, not ascending), causal and not.  Packed batches: requests with
different query and key counts, a request without query tokens, one without
keys (its rows see nothing), tokens outside every request (zero gradients),
GQA, causal / window / softcap, softmax1 sink gradients summed over the
requests, and a batch without requests.  Sparsemax draws keep every score
1e-4 clear of its row's threshold, as in the padded backward tests."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
from oracle import (attention_backward, attention_forward, varlen_attention_backward,
                    varlen_attention_forward)

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")
TOL = {torch.float32: 2e-4, torch.bfloat16: 1.5e-2}  # times max |reference|


def _assert_close(name, got, want, dtype, where):
    got = got.double().cpu().numpy()
    err = np.abs(got - want).max() if got.size else 0.0
    scale = max(np.abs(want).max() if want.size else 0.0, 1e-6)
    assert err <= TOL[dtype] * scale, f"{where} {name}: {err:.3e} vs {scale:.3e}"


def _clear(det, st):
    return all(len(z) == 0 or np.min(np.abs(np.asarray(z) - st[r, 0])) > 1e-4
               for r, (idx, p, z) in enumerate(det))


# --------------------------------------------------------------------------
# block masks

def _block_mask(seed, B, Hm, Lq, Lk, bq, bk, p=0.6):
    """Random lists: ascending used entries, plus a query block with no list
    and lists that hold ignored entries (out of range, not ascending)."""
    g = np.random.default_rng(seed)
    nqb, nkb = -(-Lq // bq), -(-Lk // bk)
    m = nkb + 2
    num = np.zeros((B, Hm, nqb), dtype=np.int32)
    idx = np.full((B, Hm, nqb, m), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hm):
            for r in range(nqb):
                c = np.nonzero(g.random(nkb) < p)[0].tolist()
                if (b + h + r) % 3 == 1 and c:
                    c = c[:1] + [nkb + 5] + [c[0]] + c[1:]  # out of range, then a repeat
                num[b, h, r] = len(c)
                idx[b, h, r, :len(c)] = c
    num[0, 0, min(1, nqb - 1)] = 0
    return num, idx


def _check_bm(norm, dtype, D, causal, bq, bk, Hm, seed, sinks=None, shape=(2, 4, 2, 70, 90)):
    B, Hq, Hkv, Lq, Lk = shape
    scaling = 1.0 / math.sqrt(D)
    num, idx = _block_mask(seed, B, Hm, Lq, Lk, bq, bk)
    bm_np = (num, idx, bq, bk)
    for s in range(seed, seed + 20):
        g = torch.Generator().manual_seed(s)
        q, k, v, do = [torch.randn(*sh, generator=g).to(dtype) for sh in
                       ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D), (B, Hq, Lq, D))]
        if norm != "sparsemax":
            break
        rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Lq)]
        _, st, det = attention_forward(q, k, v, norm, causal, 0, 0.0, scaling, rows=rows,
                                       return_probs=True, block_mask=bm_np)
        if _clear(det, st):
            break
    else:
        pytest.fail("no draw clear of the support edges")
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    bm = (torch.from_numpy(num).cuda(), torch.from_numpy(idx).cuda(), bq, bk)
    sd = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device="cuda")
    assert apn.attn_bwd_path(qd, kd, vd, dod, normalizer=norm, causal=causal, scaling=scaling,
                             sinks=sd, block_mask=bm) == "bwd_per_row"
    st = torch.empty(B, Hq, Lq, 2, device="cuda")
    apn.attn_fwd(qd, kd, vd, None, st, normalizer=norm, causal=causal, scaling=scaling, sinks=sd,
                 block_mask=bm)
    dq, dk, dv, ds = apn.attn_bwd(qd, kd, vd, dod, st, normalizer=norm, causal=causal,
                                  scaling=scaling, sinks=sd, sink_grad=sinks is not None,
                                  block_mask=bm)
    torch.cuda.synchronize()
    ref = attention_backward(q, k, v, do, norm, causal, 0, 0.0, scaling, sinks=sinks,
                             block_mask=bm_np)
    where = f"block mask {norm} {dtype} D{D} bq{bq} bk{bk} heads{Hm} causal{causal}"
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _assert_close(name, got, want, dtype, where)
    if sinks is not None:
        _assert_close("dsinks", ds, ref[3], dtype, where)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk,Hm", [(16, 16, 1), (32, 64, 4), (128, 128, 1)],
                         ids=["b16x16_shared", "b32x64_per_head", "b128x128_shared"])
def test_block_mask(norm, dtype, D, causal, bq, bk, Hm):
    _check_bm(norm, dtype, D, causal, bq, bk, Hm, 700 + bq + bk + D)


def test_block_mask_sink_gradients():
    _check_bm("softmax1", torch.float32, 64, True, 16, 32, 4, 750, sinks=[0.5, -1.0, 2.0, 0.0])


@pytest.mark.parametrize("norm", NORMS)
def test_block_mask_ragged_blocks(norm):
    # block sizes that divide neither length; head dim 256
    _check_bm(norm, torch.bfloat16, 256, True, 24, 40, 1, 760, shape=(1, 2, 1, 130, 170))


# --------------------------------------------------------------------------
# packed variable-length batches

def _cu(lens, total):
    c = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert c[-1] <= total
    return c


def _check_varlen(norm, dtype, D, causal, window, cap, seed, q_lens, k_lens, Hq=4, Hkv=2,
                  extra_q=3, extra_k=2, sinks=None):
    cq, ck = _cu(q_lens, sum(q_lens) + extra_q), _cu(k_lens, sum(k_lens) + extra_k)
    tq, tk = int(cq[-1]) + extra_q, int(ck[-1]) + extra_k  # tokens past the last request
    scaling = 1.0 / math.sqrt(D)
    for s in range(seed, seed + 20):
        g = torch.Generator().manual_seed(s)
        q, k, v, do = [torch.randn(*sh, generator=g).to(dtype) for sh in
                       ((tq, Hq, D), (tk, Hkv, D), (tk, Hkv, D), (tq, Hq, D))]
        if norm != "sparsemax":
            break
        ok = True
        for r in range(len(q_lens)):
            if q_lens[r] == 0:
                continue
            tr = lambda x, a, b_: x[a:b_].transpose(0, 1)[None]
            rows = [(0, h, i) for h in range(Hq) for i in range(q_lens[r])]
            _, st, det = attention_forward(tr(q, cq[r], cq[r + 1]), tr(k, ck[r], ck[r + 1]),
                                           tr(v, ck[r], ck[r + 1]), norm, causal, window, cap,
                                           scaling, rows=rows, return_probs=True)
            ok = ok and _clear(det, st)
        if ok:
            break
    else:
        pytest.fail("no draw clear of the support edges")
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    sd = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device="cuda")
    max_q = max(q_lens) if q_lens else 0
    st = torch.empty(Hq, tq, 2, device="cuda")
    apn.attn_fwd_varlen(qd, kd, vd, cqd, ckd, max_q, None, st, normalizer=norm, causal=causal,
                        window=window, softcap=cap, scaling=scaling, sinks=sd)
    # garbage where no request writes: the backward must not read it
    dq0 = torch.full_like(qd, float("nan"))
    dk0 = torch.full_like(kd, float("nan"))
    dv0 = torch.full_like(vd, float("nan"))
    dq, dk, dv, ds = apn.attn_bwd_varlen(qd, kd, vd, dod, st, cqd, ckd, max_q, normalizer=norm,
                                         causal=causal, window=window, softcap=cap,
                                         scaling=scaling, sinks=sd, sink_grad=sinks is not None,
                                         dq=dq0, dk=dk0, dv=dv0)
    torch.cuda.synchronize()
    ref = varlen_attention_backward(q, k, v, do, cq, ck, norm, causal, window, cap, scaling,
                                    sinks=sinks)
    where = f"varlen {norm} {dtype} D{D} causal{causal} window{window} cap{cap}"
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert torch.isfinite(got).all(), f"{where} {name}: non-finite values"
        _assert_close(name, got, want, dtype, where)
    assert (dq[cq[-1]:] == 0).all() and (dk[ck[-1]:] == 0).all() and (dv[ck[-1]:] == 0).all()
    if sinks is not None:
        _assert_close("dsinks", ds, ref[3], dtype, where)


Q_LENS, K_LENS = (37, 0, 1, 90, 20, 64), (50, 9, 33, 90, 0, 150)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128)])
@pytest.mark.parametrize("causal,window,cap", [(False, 0, 0.0), (True, 0, 0.0), (True, 16, 0.0),
                                               (True, 0, 5.0)])
def test_varlen(norm, dtype, D, causal, window, cap):
    _check_varlen(norm, dtype, D, causal, window, cap, 800 + D, Q_LENS, K_LENS)


def test_varlen_sink_gradients():
    _check_varlen("softmax1", torch.float32, 64, True, 0, 0.0, 850, Q_LENS, K_LENS,
                  sinks=[0.5, -1.0, 2.0, 0.0])
    _check_varlen("softmax1", torch.bfloat16, 128, True, 0, 0.0, 851, Q_LENS, K_LENS,
                  sinks=[1.5, 0.0, -0.5, 3.0])


@pytest.mark.parametrize("norm", NORMS)
def test_varlen_gqa8_d256(norm):
    _check_varlen(norm, torch.bfloat16, 256, True, 0, 0.0, 860, (5, 70), (40, 70), Hq=8, Hkv=1)


def test_varlen_no_requests():
    # no request: every gradient is zero, the sink gradient too
    q = torch.randn(10, 4, 64, device="cuda")
    k = torch.randn(12, 2, 64, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.zeros(4, 10, 2, device="cuda")
    dq, dk, dv, ds = apn.attn_bwd_varlen(q, k, k, q, st, cu, cu, 0, normalizer="softmax1",
                                         dq=torch.full_like(q, float("nan")),
                                         dk=torch.full_like(k, float("nan")),
                                         dv=torch.full_like(k, float("nan")), sink_grad=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, ds):
        assert (t == 0).all()


def test_varlen_matches_padded_backward():
    # one request covering the whole packed batch is the padded backward of
    # a batch of one: both GPU paths agree to the fp32 bar
    g = torch.Generator().manual_seed(870)
    Hq, Hkv, L, D = 4, 2, 77, 64
    q, do = (torch.randn(L, Hq, D, generator=g).cuda() for _ in range(2))
    k, v = (torch.randn(L, Hkv, D, generator=g).cuda() for _ in range(2))
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    st = torch.empty(Hq, L, 2, device="cuda")
    apn.attn_fwd_varlen(q, k, v, cu, cu, L, None, st, normalizer="entmax15", causal=True)
    got = apn.attn_bwd_varlen(q, k, v, do, st, cu, cu, L, normalizer="entmax15", causal=True)
    pad = lambda t: t.transpose(0, 1)[None].contiguous()
    st2 = torch.empty(1, Hq, L, 2, device="cuda")
    apn.attn_fwd(pad(q), pad(k), pad(v), None, st2, normalizer="entmax15", causal=True)
    want = apn.attn_bwd(pad(q), pad(k), pad(v), pad(do), st2, normalizer="entmax15", causal=True)
    torch.cuda.synchronize()
    for a, b in zip(got[:3], want[:3]):
        err = (a - b[0].transpose(0, 1)).abs().max().item()
        assert err <= 2e-4 * b.abs().max().item(), err
