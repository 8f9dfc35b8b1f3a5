"""Gradients of the attention forward, in float64.

Test infrastructure (see ``oracle/__init__``).  The pages' kernels all come
with a fused backward that recomputes the probabilities from the saved row
statistics ("HF Attention Normalizers", "Important Limitations": softmax1
saves row max and denominator and recomputes P in backward; the sparse
kernels save one threshold per row and recompute tiles in backward).  This
is the plain chain rule of the forward in ``oracle.attention``, row by row:

  forward   raw_ij = q_i . k_j,  s_ij = scaling * raw_ij (softcap: cap *
            tanh(scaling * raw_ij / cap)),  p_i = N(s_i over the allowed
            keys),  out_i = sum_j p_ij v_j
  backward  dV_j  += p_ij dO_i
            dP_ij  = dO_i . v_j
            ds_ij  = the normalizer's Jacobian (transposed) applied to dP_i:
              softmax / softmax1:  p_ij (dP_ij - sum_k p_ik dP_ik)
                (softmax1's virtual key has value 0, so its dP is 0)
              sparsemax:  on the support S, dP_ij - mean_{k in S} dP_ik; else 0
                (p = s - tau on S with sum p = 1 fixed, so d tau = mean ds)
              1.5-entmax, z = s / 2, p = (z - tau)^2 on S:  with u = sqrt(p),
                u_ij (dP_ij - sum_k u_ik dP_ik / sum_k u_ik) on S; else 0
                (dp = 2u (dz - d tau), sum dp = 0 gives d tau = sum u dz / sum u,
                and dz = ds / 2)
            draw_ij = ds_ij * scaling * (1 - tanh^2(scaling raw_ij / cap))
                      (without softcap: ds_ij * scaling)
            dQ_i  += draw_ij k_j,   dK_j += draw_ij q_i
  grouped-query attention: dK, dV of a key/value head sum over its G query
  heads.  softmax1 with learned sinks b_h: d b_h = -sum_i p_sink,i sum_k p_ik
  dP_ik, p_sink,i = exp(b_h - m_i) / l_i (the virtual key's weight).
Masked pairs take no part in any sum.
"""

import math

import numpy as np

from .attention import _as_f64, _check_params
from .masks import allowed_mask, block_mask_allowed
from .normalizers import normalize_row


def attention_backward(q, k, v, dout, normalizer, causal=False, window=0, softcap=0.0,
                       scaling=None, sinks=None, block_mask=None):
    """dq [B,Hq,Lq,D], dk, dv [B,Hkv,Lk,D] (float64) and, for softmax1 with
    ``sinks``, dsinks [Hq] (else None), for upstream gradient ``dout``."""
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    G = Hq // Hkv
    if scaling is None:
        scaling = 1.0 / math.sqrt(D)
    _check_params(normalizer, causal, window, softcap, scaling)
    base = allowed_mask(Lq, Lk, causal, window)
    if block_mask is not None:
        bm_num, bm_idx, bq, bk = block_mask
        bm_num = np.asarray(_as_f64(bm_num)).astype(np.int64)
        bm_idx = np.asarray(_as_f64(bm_idx)).astype(np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.zeros(Hq) if (normalizer == "softmax1" and sinks is not None) else None
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            mask = base
            if block_mask is not None:
                hm = 0 if bm_num.shape[1] == 1 else h
                mask = base & block_mask_allowed(Lq, Lk, bm_num[b, hm], bm_idx[b, hm], bq, bk)
            raw = q[b, h] @ k[b, kv].T
            if softcap > 0:
                t = np.tanh(scaling * raw / softcap)
                s = softcap * t
                dsdraw = scaling * (1.0 - t * t)
            else:
                s = scaling * raw
                dsdraw = np.full_like(raw, scaling)
            for i in range(Lq):
                idx = np.nonzero(mask[i])[0]
                if idx.size == 0:
                    continue
                sink = None if sinks is None else float(sinks[h])
                p, st0, st1 = normalize_row(normalizer, s[i, idx], sink)
                dP = v[b, kv, idx] @ dout[b, h, i]
                if normalizer in ("softmax", "softmax1"):
                    delta = float(p @ dP)
                    ds = p * (dP - delta)
                    if dsinks is not None:
                        dsinks[h] -= math.exp(sink - st0) / st1 * delta
                elif normalizer == "sparsemax":
                    sup = p > 0
                    ds = np.where(sup, dP - dP[sup].mean(), 0.0)
                else:
                    u = np.sqrt(p)
                    sup = p > 0
                    ds = np.where(sup, u * (dP - (u @ dP) / u.sum()), 0.0)
                draw = ds * dsdraw[i, idx]
                dq[b, h, i] += draw @ k[b, kv, idx]
                dk[b, kv, idx] += np.outer(draw, q[b, h, i])
                dv[b, kv, idx] += np.outer(p, dout[b, h, i])
    return dq, dk, dv, dsinks


def varlen_attention_backward(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, normalizer,
                              causal=False, window=0, softcap=0.0, scaling=None, sinks=None):
    """Gradients of ``varlen_attention_forward`` ("HF Attention Normalizers",
    "Packed Variable-Length Attention": the packed path has a full backward).

    q, dout [total_q, Hq, D]; k, v [total_k, Hkv, D]; request r owns query
    tokens cu_seqlens_q[r]..cu_seqlens_q[r+1] and key tokens
    cu_seqlens_k[r]..cu_seqlens_k[r+1] and is differentiated as a batch entry
    of its own (``attention_backward`` on its slices).  Returns dq [total_q,
    Hq, D], dk, dv [total_k, Hkv, D] (tokens outside every request: 0) and,
    for softmax1 with ``sinks``, dsinks [Hq] summed over the requests."""
    q, k, v, dout = (_as_f64(x) for x in (q, k, v, dout))
    cq = [int(x) for x in np.asarray(cu_seqlens_q)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k)]
    Hq = q.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.zeros(Hq) if (normalizer == "softmax1" and sinks is not None) else None
    tr = lambda x: np.transpose(x, (1, 0, 2))[None]
    for r in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[r], cq[r + 1], ck[r], ck[r + 1]
        if q1 == q0:
            continue
        g = attention_backward(tr(q[q0:q1]), tr(k[k0:k1]), tr(v[k0:k1]), tr(dout[q0:q1]),
                               normalizer, causal, window, softcap, scaling, sinks=sinks)
        dq[q0:q1] += np.transpose(g[0][0], (1, 0, 2))
        dk[k0:k1] += np.transpose(g[1][0], (1, 0, 2))
        dv[k0:k1] += np.transpose(g[2][0], (1, 0, 2))
        if dsinks is not None:
            dsinks += g[3]
    return dq, dk, dv, dsinks
