"""The four normalizers, on one row of allowed scores, in float64.

Test infrastructure (see ``oracle/__init__``).  Each function takes a 1-D
float64 array ``s`` holding the scores of the keys a query may attend to (masked
keys are simply absent) and returns ``(p, stat0, stat1)``:

* ``p``     -- the weights over those keys (same length as ``s``),
* ``stat0``, ``stat1`` -- the per-row statistics a fused forward keeps:
  (row max m, denominator l) for the softmax family, (threshold tau, support
  size k) for the sparse pair ("HF Attention Normalizers", "Important
  Limitations": the online softmax1 kernel saves row max and denominator, the
  sparse kernels save one threshold per query row).

Empty rows (every key masked) give p = [] and the statistics
softmax (-inf, 0), softmax1 (0, 1), sparse (+inf, 0).  The pages say nothing
about empty rows; these are the values the definitions give when the sum runs
over no keys (softmax1 keeps only its "+1").
"""

import math

import numpy as np

NORMALIZERS = ("softmax", "softmax1", "sparsemax", "entmax15")


def softmax_row(s):
    """Plain softmax, ``exp(s_i) / sum_j exp(s_j)``.

    Source: "HF Attention Normalizers", "Supported Normalizers" (the
    "vanilla / softmax" baseline).  Evaluated with the row max subtracted.
    Pinned by: PyTorch fp64 SDPA (math path) and sum-to-one.
    """
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0:
        return np.zeros(0), -math.inf, 0.0
    m = float(np.max(s))
    e = np.exp(s - m)
    l = float(np.sum(e))
    return e / l, m, l


def softmax1_row(s, sink=0.0):
    """softmax1 (Softmax-N with n = 1): ``exp(s_i) / (1 + sum_j exp(s_j))``.

    Source: "HF Attention Normalizers", "Supported Normalizers" (the formula)
    and "Important Limitations" (the online kernel treats the "+1" as a
    virtual key with logit 0 and value 0, and saves row max and denominator).

    ``sink`` generalises the virtual key's logit from 0 to a learned per-head
    value b ("Attention variants: what to open up, and how far", "What cannot
    be drawn today": attention sinks add one learned per-head term to the
    softmax's denominator): ``exp(s_i) / (exp(b) + sum_j exp(s_j))``.

    Stabilised with ``m = max(b, max_j s_j)``: both numerator and denominator
    are multiplied by ``exp(-m)``, so ``l = exp(b - m) + sum_j exp(s_j - m)``.
    Masked keys are absent; the virtual key is not a key and always stays.
    Pinned by: the closed form evaluated directly, the appended zero-key /
    zero-value identity through PyTorch fp64 SDPA, 1/(n+1) on zero rows, and
    (sink) plain softmax over the row extended by the sink logit, and the limit
    b -> -inf equal to softmax.
    """
    s = np.asarray(s, dtype=np.float64)
    b = float(sink)
    if s.size == 0:
        return np.zeros(0), b, 1.0
    m = max(b, float(np.max(s)))
    e = np.exp(s - m)
    l = math.exp(b - m) + float(np.sum(e))
    return e / l, m, l


def sparsemax_row(s):
    """sparsemax: the Euclidean projection of s onto the probability simplex.

    Source: "HF Attention Normalizers", "Supported Normalizers" (a sparse
    probability transform with exact zeros) and "Important Limitations" (one
    threshold per query row).  Written as ``p = max(z - tau, 0)`` with z = s and
    tau fixed by ``sum(p) = 1``.

    Sort-based exact solution (Martins & Astudillo, 2016): sort z in
    descending order; for each k the threshold of the top-k set is
    ``tau_k = (sum_{r<=k} z_(r) - 1) / k``; the support size is the largest k
    with ``z_(k) > tau_k``.  Returns (p, tau, k).
    Pinned by: exhaustive support enumeration on rows of length <= 8, fp64
    bisection, the two-element closed form, uniform and one-hot cases.
    """
    z = np.asarray(s, dtype=np.float64)
    n = z.size
    if n == 0:
        return np.zeros(0), math.inf, 0
    zs = np.sort(z)[::-1]
    csum = np.cumsum(zs)
    ks = np.arange(1, n + 1, dtype=np.float64)
    tau_k = (csum - 1.0) / ks
    ok = zs > tau_k
    k = int(np.nonzero(ok)[0].max()) + 1  # ok[0] always holds: z_(1) > z_(1) - 1
    tau = float(tau_k[k - 1])
    if k < n:
        # the element just outside must not exceed the threshold
        assert zs[k] <= tau + 1e-12 * max(1.0, abs(tau)), "sparsemax support inconsistent"
    p = np.maximum(z - tau, 0.0)
    # report the size of the support p actually has (they differ only when an
    # element lies within fp64 rounding of tau)
    return p, tau, int(np.count_nonzero(p))


def entmax15_row(s):
    """1.5-entmax: ``p = max(s/2 - tau, 0)**2`` with tau fixed by ``sum(p) = 1``.

    Source: "HF Attention Normalizers", "Supported Normalizers" (1.5-entmax,
    sparse, between softmax and sparsemax) and "Important Limitations" (one
    threshold per query row).  alpha-entmax with alpha = 1.5 is
    ``[(alpha - 1) s - tau]_+^(1/(alpha-1))``, i.e. z = s/2 and the square;
    tau lives in the z = s/2 domain.

    Sort-based exact solution (Peters, Niculae & Martins, 2019): sort z
    descending; for the top-k set take its mean mu_k and
    ``delta_k = (1 - sum_{r<=k} (z_(r) - mu_k)^2) / k``; where delta_k >= 0 the
    set's threshold is ``tau_k = mu_k - sqrt(delta_k)``; the support size is
    the largest such k with ``z_(k) > tau_k``.  Returns (p, tau, k).
    Pinned by: exhaustive support enumeration on rows of length <= 8, fp64
    bisection, the two-element closed form, uniform and one-hot cases.
    """
    z = np.asarray(s, dtype=np.float64) / 2.0
    n = z.size
    if n == 0:
        return np.zeros(0), math.inf, 0
    zs = np.sort(z)[::-1]
    ks = np.arange(1, n + 1, dtype=np.float64)
    # work with y = z - z_(1) <= 0 so the running sums stay small
    y = zs - zs[0]
    sy = np.cumsum(y)
    syy = np.cumsum(y * y)
    mu = zs[0] + sy / ks
    # sum of squared deviations of the top-k set from its own mean:
    # sum_r (y_r - ybar_k)^2 = sum_r y_r^2 - k * ybar_k^2
    ss = syy - sy * sy / ks
    delta = (1.0 - ss) / ks
    valid = delta >= 0.0
    tau_k = np.where(valid, mu - np.sqrt(np.where(valid, delta, 0.0)), np.inf)
    ok = valid & (zs > tau_k)
    k = int(np.nonzero(ok)[0].max()) + 1  # k = 1 always qualifies: tau_1 = z_(1) - 1
    tau = float(tau_k[k - 1])
    if k < n:
        assert zs[k] <= tau + 1e-12 * max(1.0, abs(tau)), "entmax15 support inconsistent"
    p = np.maximum(z - tau, 0.0) ** 2
    return p, tau, int(np.count_nonzero(z > tau))


_ROW_FUNCS = {
    "softmax": softmax_row,
    "softmax1": softmax1_row,
    "sparsemax": sparsemax_row,
    "entmax15": entmax15_row,
}


def normalize_row(name, s, sink=None):
    """Dispatch by normalizer name (one of ``NORMALIZERS``); ``sink`` (a
    learned sink logit) applies to softmax1 only."""
    try:
        fn = _ROW_FUNCS[name]
    except KeyError:
        raise ValueError(f"unknown normalizer {name!r}") from None
    if sink is not None:
        if name != "softmax1":
            raise ValueError("a sink logit applies to softmax1 only")
        return fn(s, sink)
    return fn(s)
