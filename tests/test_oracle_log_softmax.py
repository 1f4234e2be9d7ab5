"""Pins of the oracle's log-softmax over a row's candidates
(``oracle.log_softmax_candidates``, ``oracle.top_m_log_softmax``).

The values are fixed by the mathematics, not by the oracle's own formula:
closed forms (one candidate, n equal candidates, two candidates through
log1p), a 50-digit decimal evaluation on random rows, the invariants of a
softmax (the probabilities sum to 1, an exact common shift changes nothing,
order is kept), and the link to the pinned ``top_m`` and ``masked_logits``.
A dropped max shift overflows at logits of 1000, a wrong sign or a missing
log breaks the closed forms, and fp32 accumulation, or log(1 + T) where the
largest candidate dominates, misses the 50-digit values by far more than
one fp32 step.
"""

import decimal
import math

import numpy as np
import pytest

import oracle
from workloads import make_random


def ulps(a, b):
    """Distance in fp32 steps between two fp32 arrays of finite values."""
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_single_candidate_has_log_probability_zero():
    for v in (0.0, -3.5, 1000.0, -1000.0, 1e30):
        assert oracle.log_softmax_candidates([v]).tolist() == [0.0]


@pytest.mark.parametrize("n", [2, 3, 10, 1000, 4096])
@pytest.mark.parametrize("v", [0.0, 7.25, 1000.0, -1000.0])
def test_equal_candidates_share_minus_log_n(n, v):
    got = oracle.log_softmax_candidates(np.full(n, v, dtype=np.float32))
    want = np.float32(-math.log(n))
    assert np.all(ulps(got, np.full(n, want)) <= 1), (got[:3], want)


@pytest.mark.parametrize("a,b", [(0.0, -1.0), (3.0, 2.5), (100.0, 80.0), (-5.0, -5.0), (1000.0, 999.0)])
def test_two_candidates_closed_form(a, b):
    got = oracle.log_softmax_candidates(np.array([a, b], dtype=np.float32))
    # a >= b: log p_a = -log(1 + e^(b-a)), log p_b = (b - a) + log p_a
    la = -math.log1p(math.exp(b - a))
    lb = (b - a) + la
    assert np.all(ulps(got, np.array([la, lb], dtype=np.float32)) <= 1), (got, la, lb)


def _decimal_log_softmax(x):
    """log p_i = x_i - ln(sum_c e^(x_c)) at 50 significant digits, then the
    nearest float64 and its nearest fp32."""
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        xd = [decimal.Decimal(float(v)) for v in x]
        lse = sum(v.exp() for v in xd).ln()
        return np.array([float(v - lse) for v in xd], dtype=np.float64).astype(np.float32)


def test_high_precision_evaluation_on_random_rows():
    rng = np.random.default_rng(5)
    worst = 0
    exact = total = 0
    for n in (1, 2, 7, 64, 500, 3000):
        for scale in (0.01, 1.0, 8.0, 60.0):
            x = (rng.standard_normal(n) * scale).astype(np.float32)
            got = oracle.log_softmax_candidates(x)
            want = _decimal_log_softmax(x)
            d = ulps(got, want)
            worst = max(worst, int(d.max()))
            exact += int((d == 0).sum())
            total += n
    assert worst <= 1
    assert exact >= 0.99 * total


def test_probabilities_sum_to_one_and_order_is_kept():
    rng = np.random.default_rng(6)
    for n in (3, 100, 4000):
        x = (rng.standard_normal(n) * 4).astype(np.float32)
        lp = oracle.log_softmax_candidates(x).astype(np.float64)
        assert abs(np.exp(lp).sum() - 1.0) < n * 2.0 ** -22
        o = np.argsort(x, kind="stable")
        assert np.all(np.diff(lp[o]) >= 0)


def test_exact_common_shift_changes_nothing():
    rng = np.random.default_rng(7)
    # quarter-integers below 2^10 plus a power of two stay exact in fp32
    x = (rng.integers(-2000, 2000, 300) / 4.0).astype(np.float32)
    for c in (1.0, 64.0, 1024.0, -512.0):
        y = (x + np.float32(c)).astype(np.float32)
        assert np.array_equal(y - np.float32(c), x)
        assert np.all(ulps(oracle.log_softmax_candidates(y), oracle.log_softmax_candidates(x)) <= 1)


@pytest.mark.parametrize("ragged", [False, True])
def test_top_m_log_softmax_agrees_with_top_m_and_the_masked_row(ragged):
    w = make_random(91, d=64, V=1024, Nc=16, dtype="bf16", rows=4, ragged=ragged)
    K, m = 2, 8
    tok, lp = oracle.top_m_log_softmax(w.h, w.C, w.E, w.offsets, w.tos, K, m, "bf16")
    tok_m, val_m = oracle.top_m(w.h, w.C, w.E, w.offsets, w.tos, K, m, "bf16")
    assert np.array_equal(tok, tok_m)
    M, _ = oracle.masked_logits(w.h, w.C, w.E, w.offsets, w.tos, K, "bf16")
    for b in range(w.h.shape[0]):
        fin = np.isfinite(M[b])
        row = M[b][fin]
        full = oracle.log_softmax_candidates(row)
        by_token = dict(zip(np.nonzero(fin)[0].tolist(), full.tolist()))
        n = int((tok[b] >= 0).sum())
        assert n == min(m, int(fin.sum()))
        assert [by_token[t] for t in tok[b, :n].tolist()] == lp[b, :n].tolist()
        assert np.all(np.isneginf(lp[b, n:]))
        # differences of log-probabilities are differences of logits
        d_lp = lp[b, 0].astype(np.float64) - lp[b, n - 1].astype(np.float64)
        d_l = val_m[b, 0].astype(np.float64) - val_m[b, n - 1].astype(np.float64)
        assert abs(d_lp - d_l) <= 4 * 2.0 ** -23 * max(1.0, abs(lp[b, n - 1]))


def test_a_row_of_candidates_fitting_in_m_sums_to_one():
    w = make_random(92, d=64, V=512, Nc=32, dtype="bf16", rows=3, ragged=True)
    tok, lp = oracle.top_m_log_softmax(w.h, w.C, w.E, w.offsets, w.tos, 1, 32, "bf16")
    for b in range(3):
        n = int((tok[b] >= 0).sum())
        if n < 32:   # every candidate of the row is listed
            assert abs(np.exp(lp[b, :n].astype(np.float64)).sum() - 1.0) < 1e-5
