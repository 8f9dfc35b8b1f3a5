"""fp64 CPU oracle for attention with a pluggable normalizer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or link anything under ``oracle/``.  The only
callers are ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``.  The oracle shares no code with the GPU path: no kernels,
headers, helpers, tables or pre-/post-processing.  Inputs reach it as plain
tensors/arrays from the seeded generators in ``workloads/``.

What it computes (the forward the pages describe)::

    out = N(mask(softcap(scaling * Q K^T))) V        (grouped-query attention)

* N is softmax, softmax1, sparsemax or 1.5-entmax
  ("HF Attention Normalizers", section "Supported Normalizers").
* softcap is ``cap * tanh(score / cap)``
  ("Attention variants: what to open up, and how far", parameter table of
  "What the engine does today").
* the mask is causal and/or a sliding window ("attention interface",
  "flexattention patterns"; "tensorplay.nn.attention", create_mask example),
  plus the per-sequence length of a paged KV cache
  ("HF Attention Normalizers", "Differentiable Paged Attention"), or the
  per-request ranges of a packed variable-length batch (same page, "Packed
  Variable-Length Attention").

Every floating-point step runs in float64.  Pins: see ``tests/test_oracle_*.py``.
Parity status of each function is stated in its docstring; all are pinned.
"""

from .masks import allowed_mask, kv_range
from .normalizers import (
    NORMALIZERS,
    softmax_row,
    softmax1_row,
    sparsemax_row,
    entmax15_row,
    normalize_row,
)
from .attention import (attention_forward, paged_attention_forward, gather_paged_kv,
                        varlen_attention_forward)
from .backward import attention_backward, varlen_attention_backward

__all__ = [
    "allowed_mask",
    "kv_range",
    "NORMALIZERS",
    "softmax_row",
    "softmax1_row",
    "sparsemax_row",
    "entmax15_row",
    "normalize_row",
    "attention_forward",
    "paged_attention_forward",
    "gather_paged_kv",
    "varlen_attention_forward",
    "attention_backward",
    "varlen_attention_backward",
]
