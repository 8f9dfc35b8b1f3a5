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
* "HF Attention Normalizers", "Important Limitations": explicit full-block
  CSR masks (FlexAttention's ``BlockMask.from_kv_blocks`` with a no-op
  mask_mod): per query block, a list of key blocks whose keys are all kept.

Readings taken where the pages are silent: a window is only defined together
with causal masking (the page defines it as causal AND distance < W), so a
window without causal is rejected.  A block mask restricts the keys further:
a pair counts when its key block is listed AND the causal / window / length
rules keep it.  List entries are taken in order; one outside the key-block
range or not above its predecessor is ignored, and the count is clamped to
the list length (FlexAttention's lists are ascending and in range).
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


def block_mask_allowed(lq, lk, num_blocks, indices, block_q, block_k):
    """Boolean [lq, lk] of one (batch, head): key j is kept for query i iff
    the key block j // block_k is a used entry of query block i // block_q's
    list (``num_blocks[r]`` entries of ``indices[r]``)."""
    if block_q <= 0 or block_k <= 0:
        raise ValueError("block sizes must be > 0")
    nkb = -(-lk // block_k)
    nqb = -(-lq // block_q)
    blocks = np.zeros((nqb, nkb), dtype=bool)
    for r in range(nqb):
        n = min(max(int(num_blocks[r]), 0), len(indices[r]))
        prev = None
        for e in range(n):
            c = int(indices[r][e])
            if 0 <= c < nkb and (prev is None or c > prev):
                blocks[r, c] = True
            prev = c
    rows = np.arange(lq) // block_q
    cols = np.arange(lk) // block_k
    return blocks[rows][:, cols]
