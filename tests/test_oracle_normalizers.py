"""Pins for the oracle's normalizers.

Each check is independent of the oracle's own formulas: a brute-force search
over every possible support set, bisection on the defining equation, values
fixed by the definitions (uniform, one-hot, two-element closed forms), the
softmax1 closed form evaluated directly, and library softmax.
"""

import itertools
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import entmax15_row, softmax1_row, softmax_row, sparsemax_row


# ---------------------------------------------------------------- helpers (test side)

def _brute_support(z, power):
    """Enumerate every non-empty subset S and keep the consistent one.

    For the threshold map p = max(z - t, 0)**power with sum p = 1, a subset S is
    the support iff the t solving sum_{i in S} (z_i - t)**power = 1 (with all
    z_i > t on S) also leaves every z_j outside S at or below t.
    """
    n = len(z)
    found = []
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            zs = [z[i] for i in S]
            if power == 1:
                t = (sum(zs) - 1.0) / r
            else:
                mu = sum(zs) / r
                ss = sum((x - mu) ** 2 for x in zs)
                d = (1.0 - ss) / r
                if d < 0:
                    continue
                t = mu - math.sqrt(d)
            # consistency up to fp64 rounding at the threshold
            eps = 1e-12 * max(1.0, abs(t))
            inside = all(z[i] > t - eps for i in S)
            outside = all(z[j] <= t + eps for j in range(n) if j not in S)
            if inside and outside:
                found.append((set(S), t))
    return found


def _bisect_tau(z, power, iters=200):
    """Root of sum max(z - t, 0)**power - 1 on [max z - 1, max z] by bisection."""
    lo, hi = max(z) - 1.0, max(z)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        f = sum(max(x - mid, 0.0) ** power for x in z) - 1.0
        if f > 0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _check_against_brute(z, p, tau, k, found):
    """Same threshold, and the same support away from fp64 ties at tau.

    Elements within 1e-12 of tau may land on either side depending on
    rounding (exact ties at the threshold carry zero weight either way).
    """
    S, t = found[0]
    eps = 1e-12 * max(1.0, abs(t))
    assert abs(tau - t) <= eps
    band = {i for i in range(len(z)) if abs(z[i] - t) <= eps}
    support = set(np.nonzero(p > 0)[0].tolist())
    assert support - band == S - band
    assert abs(k - len(S)) <= len(band)
    assert all(p[i] <= eps for i in band)  # weight at most |z - tau|


ROW = st.lists(st.floats(min_value=-6, max_value=6, allow_nan=False, width=64),
               min_size=1, max_size=8)


# ---------------------------------------------------------------- softmax

def test_softmax_matches_torch():
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 100):
        s = rng.normal(size=n) * 3
        p, m, l = softmax_row(s)
        want = torch.softmax(torch.tensor(s, dtype=torch.float64), 0).numpy()
        np.testing.assert_allclose(p, want, rtol=1e-13, atol=1e-15)
        assert m == s.max()
        assert math.isclose(l, np.exp(s - s.max()).sum(), rel_tol=1e-13)
        assert math.isclose(p.sum(), 1.0, rel_tol=1e-13)


def test_softmax_large_logits_stable():
    p, m, l = softmax_row(np.array([1000.0, 999.0]))
    np.testing.assert_allclose(p, [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1))])


# ---------------------------------------------------------------- softmax1

@given(ROW)
@settings(max_examples=200, deadline=None)
def test_softmax1_closed_form(row):
    # exp(x_i) / (1 + sum_j exp(x_j)) evaluated literally (|x| <= 6 cannot overflow)
    s = np.array(row)
    p, m, l = softmax1_row(s)
    e = [math.exp(x) for x in row]
    want = [x / (1.0 + sum(e)) for x in e]
    np.testing.assert_allclose(p, want, rtol=1e-12)
    assert 0.0 < p.sum() < 1.0
    # the statistics reproduce the weights: p = exp(s - m) / l
    np.testing.assert_allclose(np.exp(s - m) / l, p, rtol=1e-12)
    assert m == max(0.0, max(row))


def test_softmax1_zero_row_is_one_over_n_plus_one():
    for n in (1, 3, 10):
        p, m, l = softmax1_row(np.zeros(n))
        np.testing.assert_allclose(p, np.full(n, 1.0 / (n + 1)), rtol=1e-15)
        assert m == 0.0 and l == n + 1


def test_softmax1_is_softmax_with_a_zero_logit():
    # the "+1" as a virtual logit-0 key: softmax over [0; s] with the first entry dropped
    rng = np.random.default_rng(1)
    s = rng.normal(size=17) * 4
    p, _, _ = softmax1_row(s)
    full = torch.softmax(torch.tensor(np.concatenate([[0.0], s])), 0).numpy()
    np.testing.assert_allclose(p, full[1:], rtol=1e-13)


def test_softmax1_large_logits_stable():
    p, m, l = softmax1_row(np.array([800.0, 800.0]))
    np.testing.assert_allclose(p, [0.5, 0.5], rtol=1e-14)
    assert m == 800.0


def test_empty_rows():
    assert softmax_row(np.zeros(0))[1:] == (-math.inf, 0.0)
    assert softmax1_row(np.zeros(0))[1:] == (0.0, 1.0)
    assert sparsemax_row(np.zeros(0))[1:] == (math.inf, 0)
    assert entmax15_row(np.zeros(0))[1:] == (math.inf, 0)


# ---------------------------------------------------------------- sparsemax / entmax15

@given(ROW)
@settings(max_examples=300, deadline=None)
def test_sparsemax_vs_brute_force(row):
    z = list(row)
    found = _brute_support(z, 1)
    assert len(found) >= 1
    p, tau, k = sparsemax_row(np.array(z))
    _check_against_brute(z, p, tau, k, found)


@given(ROW)
@settings(max_examples=300, deadline=None)
def test_entmax15_vs_brute_force(row):
    s = list(row)
    z = [x / 2.0 for x in s]
    found = _brute_support(z, 2)
    assert len(found) >= 1
    p, tau, k = entmax15_row(np.array(s))
    _check_against_brute(z, p, tau, k, found)


@pytest.mark.parametrize("n,scale", [(30, 0.1), (200, 1.0), (1000, 0.3), (64, 5.0)])
def test_sparse_vs_bisection(n, scale):
    rng = np.random.default_rng(n)
    s = rng.normal(size=n) * scale
    p, tau, k = sparsemax_row(s)
    assert abs(tau - _bisect_tau(list(s), 1)) < 1e-12
    p2, tau2, k2 = entmax15_row(s)
    assert abs(tau2 - _bisect_tau(list(s / 2.0), 2)) < 1e-12


@given(st.lists(st.floats(min_value=-20, max_value=20, allow_nan=False, width=64),
                min_size=1, max_size=300))
@settings(max_examples=150, deadline=None)
def test_sparse_invariants(row):
    s = np.array(row)
    for fn, z, power in ((sparsemax_row, s, 1), (entmax15_row, s / 2.0, 2)):
        p, tau, k = fn(s)
        assert (p >= 0).all()
        assert math.isclose(p.sum(), 1.0, rel_tol=1e-10)
        # exact zeros exactly off the support {z > tau}, except where
        # (z - tau)**2 underflows to zero (z barely above tau)
        assert ((p > 0) <= (z > tau)).all()
        np.testing.assert_array_equal(p > 0, np.maximum(z - tau, 0.0) ** power > 0)
        assert k == int((z > tau).sum())
        np.testing.assert_allclose(p, np.maximum(z - tau, 0.0) ** power, rtol=0, atol=0)


def test_uniform_rows():
    for n in (1, 4, 33):
        c = 0.7
        p, tau, k = sparsemax_row(np.full(n, c))
        np.testing.assert_allclose(p, np.full(n, 1.0 / n), rtol=1e-12)
        assert k == n and math.isclose(tau, c - 1.0 / n)
        p, tau, k = entmax15_row(np.full(n, 2 * c))
        np.testing.assert_allclose(p, np.full(n, 1.0 / n), rtol=1e-13)
        assert k == n and math.isclose(tau, c - 1.0 / math.sqrt(n))


def test_one_hot_when_top_gap_at_least_one():
    s = np.array([3.0, 1.9, 2.0, -5.0])  # gap 1.0 in z for sparsemax
    p, tau, k = sparsemax_row(s)
    np.testing.assert_array_equal(p, [1.0, 0, 0, 0])
    assert k == 1
    s = np.array([6.0, 3.9, 2.0])        # gap in z = s/2 is 1.05 for entmax15
    p, tau, k = entmax15_row(s)
    np.testing.assert_array_equal(p, [1.0, 0, 0])
    assert k == 1 and tau == 2.0


@pytest.mark.parametrize("d", [0.0, 0.25, 0.5, 0.99])
def test_two_element_closed_forms(d):
    # sparsemax: p1 - p2 = d and p1 + p2 = 1
    p, tau, k = sparsemax_row(np.array([1.0 + d, 1.0]))
    np.testing.assert_allclose(p, [(1 + d) / 2, (1 - d) / 2], rtol=1e-12)
    # entmax15 in z: a^2 + (a - d)^2 = 1 with a = z1 - tau
    a = (d + math.sqrt(2.0 - d * d)) / 2.0
    p, tau, k = entmax15_row(2.0 * np.array([1.0 + d, 1.0]))
    np.testing.assert_allclose(p, [a * a, (a - d) ** 2], rtol=1e-11)
    assert math.isclose(tau, 1.0 + d - a, rel_tol=1e-14)


def test_shift_invariance_and_entmax_scale():
    rng = np.random.default_rng(5)
    s = rng.normal(size=50)
    p0, t0, _ = sparsemax_row(s)
    p1, t1, _ = sparsemax_row(s + 3.25)
    np.testing.assert_allclose(p0, p1, atol=1e-13)
    assert math.isclose(t1 - t0, 3.25, rel_tol=1e-12)
    # entmax15 acts on s/2: doubling s doubles z, so equals the map on z = s
    q0, u0, _ = entmax15_row(2.0 * s)
    q1, u1, _ = entmax15_row(2.0 * s + 1.0)
    np.testing.assert_allclose(q0, q1, atol=1e-13)
    assert math.isclose(u1 - u0, 0.5, rel_tol=1e-12)


def test_sparsemax_is_simplex_projection():
    # sparsemax(z) = argmin_{p in simplex} ||p - z||^2: no random simplex point is closer
    rng = np.random.default_rng(7)
    z = rng.normal(size=6)
    p, _, _ = sparsemax_row(z)
    best = np.sum((p - z) ** 2)
    for _ in range(2000):
        x = rng.dirichlet(np.ones(6) * 0.3)
        assert np.sum((x - z) ** 2) >= best - 1e-12


@pytest.mark.parametrize("sink", [-3.0, 0.0, 1.25, 40.0])
def test_softmax1_sink_is_softmax_of_the_extended_row(sink):
    s = np.random.default_rng(5).normal(size=9) * 3.0
    p, m, l = softmax1_row(s, sink)
    e = np.exp(np.append(s, sink) - max(sink, s.max()))
    np.testing.assert_allclose(p, (e / e.sum())[:-1], rtol=1e-14)
    assert m == max(sink, s.max())
    # literal closed form exp(s) / (exp(b) + sum exp(s)) where it cannot overflow
    if sink < 30:
        np.testing.assert_allclose(p, np.exp(s) / (math.exp(sink) + np.exp(s).sum()), rtol=1e-13)
    assert softmax1_row(np.zeros(0), sink)[1:] == (sink, 1.0)
