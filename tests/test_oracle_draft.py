"""Pins of the draft-step oracle (final RMSNorm and scaled embedding lookup).

Each check ties the oracle to something other than itself: hand-derived
values (tests/golden/draft_step.json), an exact rational evaluation of the
norm, scale invariance, signed-zero special cases.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import draft as ds
from workloads.synth import f32_to_bf16_bits as _synth_bf16

def to_bf16_bits(a):
    """Seeded test inputs as bf16 bit patterns (the workload generator's
    rounding, which is input generation, not the method)."""
    return _synth_bf16(np.asarray(a, dtype=np.float32))


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "draft_step.json")


def _bits(s):
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint16)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _hex_array(c, key, rest_key, d, dt):
    """A golden vector: "<key>_fill", a "<key>" string of repeated bit
    patterns, or a sparse "<key>" dict with the other entries "<rest_key>"."""
    if key + "_fill" in c:
        return np.full(d, int(c[key + "_fill"], 16), dtype=dt)
    v = c[key]
    if isinstance(v, dict):
        out = np.full(d, int(c.get(rest_key, "0x0"), 16), dtype=dt)
        for k, b in v.items():
            out[int(k)] = int(b, 16)
        return out
    return np.tile(np.array([int(t, 16) for t in v.split()], dtype=dt), c[key + "_repeat"])


def _case_arrays(c):
    """(x, w, expected) of a golden norm case: bf16 bit patterns, or float32
    values for "dtype": "f32"."""
    d = c["d"]
    f32 = c.get("dtype", "bf16") == "f32"
    dt = np.uint32 if f32 else np.uint16
    x = _hex_array(c, "x", "x_rest", d, dt)
    w = _hex_array(c, "w", "w_rest", d, dt)
    want = w.copy() if c["expect"] == "same as w" else _hex_array(c, "expect", "expect_rest", d, dt)
    if f32:
        x, w, want = x.view(np.float32), w.view(np.float32), want.view(np.float32)
    return x, w, want


def test_golden_rms_norm(golden):
    for c in golden["rms_norm"]:
        x, w, want = _case_arrays(c)
        dtype = c.get("dtype", "bf16")
        got = ds.rms_norm(x[None, :], w, c["eps"], dtype)[0]
        if dtype == "f32":
            got, want = got.view(np.uint32), want.view(np.uint32)
        assert np.array_equal(got, want), c["name"]


def test_sum_of_squares_is_sequential():
    """The absorbed-squares golden row: its sequential sum of squares is
    exactly 2^54 (every later square is below half a float64 spacing there),
    while the exact sum is 2^54 + 63 (1 + 2^-22 + 2^-46)."""
    x = np.full((1, 64), np.float32(1.0 + 2.0 ** -23), dtype=np.float32)
    x[0, 0] = np.float32(2.0 ** 27)
    assert ds.sum_of_squares(x, "f32")[0] == 2.0 ** 54
    # the same squares in the opposite order: the 63 small ones first
    # (63 + 63 (2^-22 + 2^-46), exact below 2^54), then 2^54 added once:
    # the exact sum rounded once, the float64 multiple of 4 nearest 2^54 + 63.000015
    assert ds.sum_of_squares(x[:, ::-1].copy(), "f32")[0] == 2.0 ** 54 + 64


@pytest.mark.parametrize("seed,d,scale", [(1, 64, 1.0), (2, 256, 1e3), (3, 192, 1e-3)])
def test_sum_of_squares_within_sequential_bound(seed, d, scale):
    """Against exact rationals: every partial sum of positive terms rounds
    once, so |ss - exact| <= (d - 1) 2^-53 exact (to first order).  Exponent-
    spread rows (a few entries 2^20 larger) exercise absorption."""
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((4, d)) * scale).astype(np.float32)
    X[:, ::17] *= np.float32(2.0 ** 20)
    got = ds.sum_of_squares(X, "f32")
    for b in range(4):
        exact = sum(Fraction(float(v)) ** 2 for v in X[b])
        err = abs(Fraction(float(got[b])) - exact)
        assert err <= Fraction(d, 2 ** 53) * exact, b


def test_golden_embedding(golden):
    for c in golden["embed"]:
        n = np.float32(c["normalizer_num"] * 2.0 ** c["normalizer_exp2"])
        assert float(n) == c["normalizer_num"] * 2.0 ** c["normalizer_exp2"]   # exact in fp32
        table = np.array([[int(c["e"], 16)]], dtype=np.uint16)
        got = ds.embed_rows(table, np.array([0]), n, "bf16")
        assert got[0, 0] == int(c["expect"], 16), c["name"]


def _bf16_of_fraction(q: Fraction) -> int:
    """bf16 bits of the exact rational q rounded to nearest, ties to even
    (normal range only)."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    m = a / Fraction(2) ** e * 128          # in [128, 256)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    if fl == 256:
        fl, e = 128, e + 1
    return sign | ((e + 127) << 7) | (fl - 128)


def _distance_to_tie(q: Fraction) -> float:
    """Relative distance of q to the nearest bf16 rounding boundary."""
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    m = a / Fraction(2) ** e * 128
    frac = m - m.numerator // m.denominator
    return float(abs(frac - Fraction(1, 2))) / 128.0


def _isqrt_fraction(v: Fraction, bits: int = 200) -> Fraction:
    """sqrt(v) to `bits` fractional bits (floor), exactly from integers."""
    scale = 1 << (2 * bits)
    n = v.numerator * scale // v.denominator
    from math import isqrt
    return Fraction(isqrt(n), 1 << bits)


@pytest.mark.parametrize("seed,d,eps", [(1, 64, 1e-6), (2, 128, 1e-6), (3, 256, 0.5), (4, 64, 0.0)])
def test_rms_norm_matches_exact_value(seed, d, eps):
    """Each bf16 output is the exact real x_k w_k / sqrt(mean x^2 + eps)
    rounded to bf16, except where that value sits within float64 noise of a
    bf16 rounding boundary (skipped: the canonical float64 steps decide)."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((3, d)) * 2.0)
    w = to_bf16_bits(1.0 + 0.25 * rng.standard_normal(d))
    got = ds.rms_norm(x, w, eps, "bf16")
    X = (x.astype(np.uint32) << 16).view(np.float32)
    W = (w.astype(np.uint32) << 16).view(np.float32)
    eps_q = Fraction(float(np.float32(eps)))
    checked = 0
    for b in range(3):
        ss = sum(Fraction(float(v)) ** 2 for v in X[b])
        s = _isqrt_fraction(ss / d + eps_q)
        for k in range(d):
            y = Fraction(float(X[b, k])) * Fraction(float(W[k])) / s
            if y == 0:
                assert got[b, k] & 0x7FFF == 0
                continue
            if _distance_to_tie(y) < 1e-12:
                continue
            assert got[b, k] == _bf16_of_fraction(y), (b, k)
            checked += 1
    assert checked > 3 * d * 0.99


@pytest.mark.parametrize("k", [-5, 3])
def test_rms_norm_scale_invariance(k):
    """With eps = 0, scaling x by 2^k changes nothing: every float64 step
    scales exactly (squares by 4^k, sqrt by 2^k, r by 2^-k)."""
    rng = np.random.default_rng(11)
    x = to_bf16_bits(rng.standard_normal((4, 192)))
    w = to_bf16_bits(rng.standard_normal(192))
    xs = x.astype(np.int32)
    nz = (xs & 0x7F80) != 0
    xs[nz] += k << 7                        # exponent shift of the normal values
    h0 = ds.rms_norm(x, w, 0.0, "bf16")
    h1 = ds.rms_norm(xs.astype(np.uint16), w, 0.0, "bf16")
    assert np.array_equal(h0, h1)


def test_rms_norm_f32_constant_row():
    d = 128
    x = np.full((1, d), -0.5, dtype=np.float32)
    w = np.random.default_rng(5).standard_normal(d).astype(np.float32)
    h = ds.rms_norm(x, w, 0.0, "f32")
    # ss = d/4, v = 1/4, r = 2, x r = -1: y = -w exactly
    assert np.array_equal(h[0], -w)


def test_rms_norm_rejects_ragged_d():
    with pytest.raises(ValueError):
        ds.rms_norm(np.zeros((1, 96), np.uint16), np.zeros(96, np.uint16), 1e-6, "bf16")


def test_embed_rows_identity_zero_and_padding():
    rng = np.random.default_rng(3)
    table = to_bf16_bits(rng.standard_normal((10, 24)))
    out = ds.embed_rows(table, np.array([7, -1, 2]), 1.0, "bf16")
    assert np.array_equal(out[0], table[7])          # times 1 is exact
    assert not out[1].any()                          # no candidate: zeros
    assert np.array_equal(out[2], table[2])
    # times 4: the exponent field grows by 2 for every normal value
    t4 = ds.embed_rows(table, np.array([5]), 4.0, "bf16")[0].astype(np.int32)
    assert np.array_equal(t4, table[5].astype(np.int32) + (2 << 7))


def test_bf16_rounding_edges():
    f = np.array([np.inf, -np.inf, np.nan, 3.4e38, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8],
                 dtype=np.float32)
    got = ds.f32_to_bf16_bits(f)
    # inf stays inf; NaN is quiet; 3.4e38 rounds past the largest finite bf16
    # to inf; halfway cases go to the even neighbour (1.0 and 1 + 2^-6)
    assert list(got) == [0x7F80, 0xFF80, 0x7FC0, 0x7F80, 0x3F80, 0x3F82]


def test_draft_step_uses_normalised_rows():
    """The draft step is the head applied to the normalised rows, and the
    embeddings are those of the tokens it picked."""
    from oracle import top_tokens
    rng = np.random.default_rng(9)
    d, Nc, vpc = 64, 16, 8
    V = Nc * vpc
    C = to_bf16_bits(rng.standard_normal((Nc, d)) / 8)
    E = to_bf16_bits(rng.standard_normal((V, d)) / 8)
    offsets = np.arange(Nc + 1) * vpc
    tos = rng.permutation(V)
    x = to_bf16_bits(rng.standard_normal((5, d)))
    w = to_bf16_bits(np.ones(d))
    table = to_bf16_bits(rng.standard_normal((V, 16)))
    h, tok, emb, sel = ds.draft_step(x, w, 1e-6, C, E, offsets, tos, 3, table, 2.0, "bf16")
    tok2, sel2, _ = top_tokens(h, C, E, offsets, tos, 3, "bf16")
    assert np.array_equal(tok, tok2) and np.array_equal(sel, sel2)
    assert np.array_equal(emb, ds.embed_rows(table, tok, 2.0, "bf16"))


def test_draft_step_hand_derived_end_to_end():
    """A whole draft step whose every output follows by hand.

    A constant row of 2.0 has mean square 4, so with a negligible eps its
    RMSNorm is exactly the weight w.  One-hot centroids make the scores the
    first coordinates of w, so the top-2 set is {2, 4}.  Every candidate
    embedding is zero except coordinate 2, where w is 1.0, so a logit is that
    coordinate's value.  Slots 9 (cluster 2) and 17 (cluster 4) tie at the
    maximum 0.9375; token_of_slot maps slot 17 to the lower token id, so it
    wins.  The normalizer 4 is a power of two, so the embedding row is the
    table row with every exponent raised by 2.
    """
    d, Nc, vpc, K = 64, 8, 4, 2
    V = Nc * vpc
    x = to_bf16_bits(np.full((1, d), 2.0))
    wv = np.zeros(d)
    wv[:8] = [0.5, 0.25, 1.0, 0.125, 0.75, 0.0, -1.0, 0.375]
    w = to_bf16_bits(wv)
    C = to_bf16_bits(np.eye(Nc, d))
    Ev = np.zeros((V, d))
    Ev[8:12, 2] = [0.5, 0.9375, 0.25, 0.125]       # cluster 2
    Ev[16:20, 2] = [0.375, 0.9375, 0.0, 0.5]       # cluster 4
    Ev[0:8, 5] = 7.0                                # clusters 0 and 1: not selected
    E = to_bf16_bits(Ev)
    offsets = np.arange(Nc + 1) * vpc
    tos = np.arange(V)[::-1].copy()                 # slot s holds token V-1-s
    table = to_bf16_bits(np.arange(V * 16).reshape(V, 16) / 64.0 + 1.0)
    h, tok, emb, sel = ds.draft_step(x, w, 1e-30, C, E, offsets, tos, K, table, 4.0, "bf16")
    assert np.array_equal(h[0], w)
    assert sel.tolist() == [[2, 4]]
    assert tok.tolist() == [V - 1 - 17]             # token 14 beats token 22 (slot 9)
    want = to_bf16_bits((np.arange(16) + (V - 1 - 17) * 16) / 64.0 * 4.0 + 4.0)
    assert np.array_equal(emb[0], want)
