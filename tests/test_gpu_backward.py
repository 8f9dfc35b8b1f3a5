"""GPU parity of the backward (attn_bwd): dq, dk, dv (and softmax1 sink
gradients) against the float64 backward oracle, from the row statistics the
GPU forward saved.  f32 and bf16 inputs, GQA, Lq != Lk, causal / window /
softcap.  bf16 at head dim 64, 128 and 256 runs the matrix-core kernels (several
key and query tiles, ragged ends, rows without keys); other cases the
per-row kernels.  Sparsemax rows are drawn so that no score lies within 1e-4 of the
row's threshold (its Jacobian jumps when a key crosses the support edge, so
a rounding-level difference there is not a parity error)."""

import math

import numpy as np
import pytest
import torch

import attention_pluggable_normalizers_amd as apn
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu
NORMS = ("softmax", "softmax1", "sparsemax", "entmax15")
TOL = {torch.float32: 2e-4, torch.bfloat16: 1.5e-2}  # times max |reference|


def _inputs(seed, B, Hq, Hkv, Lq, Lk, D, dtype):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(*s, generator=g).to(dtype) for s in
            ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D), (B, Hq, Lq, D))]


def _clear_of_edges(q, k, v, norm, causal, window, cap, scaling):
    if norm != "sparsemax":
        return True
    B, Hq, Lq, _ = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Lq)]
    _, st, det = attention_forward(q, k, v, norm, causal, window, cap, scaling, rows=rows,
                                   return_probs=True)
    return all(len(z) == 0 or np.min(np.abs(np.asarray(z) - st[r, 0])) > 1e-4
               for r, (idx, p, z) in enumerate(det))


def _check(norm, dtype, D, causal, window, cap, seed, sinks=None, shape=(2, 4, 2, 70, 90),
           use_out=False):
    B, Hq, Hkv, Lq, Lk = shape
    scaling = 1.0 / math.sqrt(D)
    for s in range(seed, seed + 20):
        q, k, v, do = _inputs(s, B, Hq, Hkv, Lq, Lk, D, dtype)
        if _clear_of_edges(q, k, v, norm, causal, window, cap, scaling):
            break
    else:
        pytest.fail("no draw clear of the support edges")
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    sd = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device="cuda")
    st = torch.empty(B, Hq, Lq, 2, device="cuda")
    out, _ = apn.attn_fwd(qd, kd, vd, None, st, normalizer=norm, causal=causal, window=window,
                          softcap=cap, scaling=scaling, sinks=sd)
    dq, dk, dv, ds = apn.attn_bwd(qd, kd, vd, dod, st, normalizer=norm, causal=causal,
                                  window=window, softcap=cap, scaling=scaling, sinks=sd,
                                  sink_grad=sinks is not None, out=out if use_out else None)
    torch.cuda.synchronize()
    ref = attention_backward(q, k, v, do, norm, causal, window, cap, scaling, sinks=sinks)
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        got = got.double().cpu().numpy()
        err = np.abs(got - want).max()
        scale = max(np.abs(want).max(), 1e-6)
        assert err <= TOL[dtype] * scale, f"{norm} {dtype} D{D} {name}: {err:.3e} vs {scale:.3e}"
    if sinks is not None:
        err = np.abs(ds.double().cpu().numpy() - ref[3]).max()
        assert err <= TOL[dtype] * max(np.abs(ref[3]).max(), 1e-6), f"dsinks {err:.3e}"


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_causal(norm, dtype, D):
    _check(norm, dtype, D, True, 0, 0.0, 100 + D)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("causal,window,cap", [(False, 0, 0.0), (True, 20, 0.0), (True, 0, 5.0)])
def test_masks_and_softcap(norm, causal, window, cap):
    _check(norm, torch.float32, 64, causal, window, cap, 200)


def test_softmax1_sink_gradients():
    _check("softmax1", torch.float32, 64, True, 0, 0.0, 300, sinks=[0.5, -1.0, 2.0, 0.0])
    _check("softmax1", torch.bfloat16, 64, True, 0, 0.0, 301, sinks=[1.5, 0.0, -0.5, 3.0])


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal,window,cap", [(False, 0, 0.0), (True, 20, 0.0), (True, 0, 5.0),
                                               (True, 150, 30.0)])
def test_mfma_masks_and_softcap(norm, D, causal, window, cap):
    _check(norm, torch.bfloat16, D, causal, window, cap, 400 + D)


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("shape", [(1, 4, 1, 200, 333), (1, 2, 2, 300, 300), (2, 2, 1, 150, 100)],
                         ids=["gqa4_lq200_lk333", "mha_300", "lq150_lk100_empty_rows"])
def test_mfma_multi_tile(norm, D, shape):
    _check(norm, torch.bfloat16, D, True, 0, 0.0, 500 + D, shape=shape)


def test_mfma_sink_gradients():
    _check("softmax1", torch.bfloat16, 128, True, 0, 0.0, 302, sinks=[0.5, -1.0, 2.0, 0.0])


@pytest.mark.parametrize("norm", NORMS)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal,window,cap", [(True, 0, 0.0), (True, 20, 0.0), (True, 0, 5.0)])
def test_with_forward_output(norm, D, causal, window, cap):
    # softmax family: the row constant from dout . out (one pass fewer);
    # the sparse normalizers ignore out
    _check(norm, torch.bfloat16, D, causal, window, cap, 600 + D, use_out=True,
           shape=(1, 4, 2, 150, 200))


def test_with_forward_output_sinks():
    _check("softmax1", torch.bfloat16, 64, True, 0, 0.0, 303, sinks=[0.5, -1.0, 2.0, 0.0],
           use_out=True)


@pytest.mark.parametrize("norm,D", [("softmax", 64), ("entmax15", 64), ("softmax1", 128),
                                    ("entmax15", 256)])
def test_mfma_key_kernel_per_kv_head(norm, D):
    # 128 x 8 (batch, kv head) pairs of one 128-key block: a grid large enough
    # that the key kernel keeps one workgroup per kv head and loops over its
    # G = 2 query heads (smaller grids split the heads and add fp32 partials)
    _check(norm, torch.bfloat16, D, True, 0, 0.0, 700 + D, shape=(128, 16, 8, 16, 128))
