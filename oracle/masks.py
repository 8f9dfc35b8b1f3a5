"""Which (query, key) pairs count.  Test infrastructure (see ``oracle/__init__``).

Sources:
* "attention interface" (transformers-v5 wiki), "flexattention patterns":
  the causal mask_mod keeps ``q_idx >= k_idx``; the sliding-window mask keeps
  ``(q >= k) and (q - k < window_size)``.
* "tensorplay.nn.attention": ``create_mask(and_masks(causal, window))`` with
  ``q_idx - kv_idx < 4`` over Q_LEN = KV_LEN = 6 gives a (1, 1, 6, 6) bool mask.
* "HF Attention Normalizers", "Packed Variable-Length Attention": causal
  attention with different query and key lengths is aligned bottom-right,
  i.e. the last query sees the last key.
* "HF Attention Normalizers", "Differentiable Paged Attention": a paged
  sequence has ``sequence_lengths[b]`` live keys; later slots are never read.

Reading taken where the pages are silent: a window is only defined together
with causal masking (the page defines it as causal AND distance < W), so a
window without causal is rejected.
"""

import numpy as np


def allowed_mask(lq, lk, causal, window=0, seq_len=None):
    """Boolean [lq, lk] matrix of the pairs a query may attend to.

    Query i sits at absolute key position ``qp = i + (L - lq)`` where L is the
    number of live keys (``seq_len`` if given, else ``lk``): bottom-right
    alignment.  Key j is allowed iff
        j < L  and  (not causal or j <= qp)  and  (window == 0 or qp - j < window).
    """
    if window and not causal:
        raise ValueError("a sliding window is only defined together with causal masking")
    if window < 0:
        raise ValueError("window must be >= 0")
    live = lk if seq_len is None else int(seq_len)
    if live > lk:
        raise ValueError("seq_len exceeds the key dimension")
    i = np.arange(lq, dtype=np.int64)[:, None]
    j = np.arange(lk, dtype=np.int64)[None, :]
    qp = i + (live - lq)
    mask = j < live
    if causal:
        mask = mask & (j <= qp)
    if window:
        mask = mask & (qp - j < window)
    return np.broadcast_to(mask, (lq, lk)).copy()


def kv_range(i, lq, live, causal, window=0):
    """[lo, hi) key interval allowed for query i (every mask row is an interval).

    Same predicate as ``allowed_mask``, solved for j.
    """
    qp = i + (live - lq)
    hi = live if not causal else min(live, qp + 1)
    hi = max(hi, 0)
    lo = 0 if not window else max(0, qp - window + 1)
    lo = min(lo, hi)
    return lo, hi
