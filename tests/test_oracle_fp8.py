"""Pins of the FP8-slab oracle (E4M3 coding, row quantisation, FP8 logits).

E4M3 decoding and rounding are pinned by hand-derived cases from the OCP
8-bit floating point specification (tests/golden/fp8_e4m3.json), the
quantisation by exact scale invariance and representable rows, the logits by
exact rationals and a brute-force argmax, and the error against the bf16
head by the bound that three mantissa bits give.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import fp8_slabs as f8
from workloads import make_random
from workloads.synth import f32_to_bf16_bits as _synth_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3.json")


def bf16(a):
    """Seeded inputs as bf16 bit patterns (the generator's rounding)."""
    return _synth_bf16(np.asarray(a, dtype=np.float32))


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_decode(golden):
    for c in golden["decode"]:
        v = f8.e4m3_decode(np.array([int(c["code"], 16)]))[0]
        if c["value"] == "nan":
            assert np.isnan(v), c
        elif c["value"] == "-0":
            assert v == 0 and np.signbit(v), c
        else:
            assert v == float(c["value"]) and not (v == 0 and np.signbit(v)), c


def test_golden_encode(golden):
    for c in golden["encode"]:
        got = f8.e4m3_encode(np.array([float(c["value"])]))[0]
        assert got == int(c["code"], 16), c


def test_decode_monotone_and_round_trip():
    codes = np.arange(0x7F, dtype=np.uint8)             # every finite positive code
    v = f8.e4m3_decode(codes)
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(f8.e4m3_encode(v), codes)
    neg = codes | 0x80
    assert np.array_equal(f8.e4m3_encode(f8.e4m3_decode(neg)), neg)


def test_encode_is_nearest():
    """Every encoded value is a nearest representable value (brute force
    over all finite codes), saturating above 448."""
    rng = np.random.default_rng(3)
    grid = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.concatenate([rng.uniform(0, 500, 4000), rng.uniform(0, 0.02, 4000),
                        np.exp2(rng.uniform(-12, 9, 4000))])
    got = f8.e4m3_decode(f8.e4m3_encode(x))
    best = np.abs(grid[None, :] - np.minimum(x, 448.0)[:, None]).min(axis=1)
    assert np.array_equal(np.abs(got - np.minimum(x, 448.0)), best)


def test_quantize_representable_row_and_scale_invariance():
    vals = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))       # 0 .. 448
    row = np.concatenate([vals, -vals[1:], np.zeros(1)])[:64 * 4]
    row = np.resize(row, 256)
    row[0] = 448.0
    bits = bf16(row)                                             # all exact in bf16
    codes, s = f8.quantize_rows(bits[None, :])
    assert s[0] == 1.0                                           # 448 / 448
    assert np.array_equal(f8.e4m3_decode(codes[0]), (bits.astype(np.uint32) << 16).view(np.float32))
    # times 2^k: the same codes, the scale times 2^k
    for k in (-20, 7):
        b2 = bits.astype(np.int32)
        nz = (b2 & 0x7F80) != 0
        b2[nz] += k << 7
        c2, s2 = f8.quantize_rows(b2.astype(np.uint16)[None, :])
        assert np.array_equal(c2, codes) and s2[0] == np.float32(2.0 ** k)


def test_quantize_zero_row():
    bits = np.zeros((1, 64), dtype=np.uint16)
    bits[0, 5] = 0x8000
    codes, s = f8.quantize_rows(bits)
    assert s[0] == 1.0 and codes[0, 0] == 0 and codes[0, 5] == 0x80


def test_fp8_logits_exact_rationals():
    rng = np.random.default_rng(5)
    d = 64
    h = bf16(rng.standard_normal(d))
    E = bf16(rng.standard_normal((40, d)) / 8)
    codes, s = f8.quantize_rows(E)
    h64 = oracle.upcast(h, "bf16")
    L = f8.fp8_chain_logits(h64, codes, s)
    Q = f8.e4m3_decode(codes)
    for j in range(40):
        exact = sum(Fraction(float(h64[k])) * Fraction(float(Q[j, k])) for k in range(d))
        exact *= Fraction(float(s[j]))
        ref = np.float32(float(exact))           # nearest fp32 of a double near it
        assert abs(float(L[j]) - float(exact)) <= abs(float(ref) - float(exact)) + \
            float(np.spacing(np.float32(abs(float(exact)))))


def test_top_tokens_full_k_is_brute_force_argmax():
    w = make_random(7, d=64, V=2048, Nc=16, dtype="bf16", rows=4)
    codes, s = f8.quantize_rows(w.E)
    tok, sel = f8.top_tokens_fp8(w.h, w.C, codes, s, w.offsets, w.tos, w.Nc)
    for b in range(4):
        L = f8.fp8_chain_logits(oracle.upcast(w.h[b], "bf16"), codes, s)
        best = L.max()
        assert tok[b] == np.asarray(w.tos)[L == best].min()
        assert sel[b].tolist() == list(range(w.Nc))


def test_error_against_bf16_head_within_bound():
    """|L_fp8 - L_bf16| <= sum_k |h_k| (2^-4 |x_k| + 2^-10 s) + fp32 roundings:
    three mantissa bits give relative error 2^-4, subnormals 2^-10 s."""
    w = make_random(8, d=128, V=4096, Nc=32, dtype="bf16", rows=6)
    codes, s = f8.quantize_rows(w.E)
    for b in range(6):
        lf, tf, _ = f8.select_and_score_fp8(w.h[b], w.C, codes, s, w.offsets, w.tos, 4)
        lb, tb, _ = oracle.select_and_score(w.h[b], w.C, w.E, w.offsets, w.tos, 4, "bf16")
        assert np.array_equal(tf, tb)
        h = np.abs(oracle.upcast(w.h[b], "bf16"))
        inv = {int(t): i for i, t in enumerate(w.tos)}
        X = np.abs(oracle.upcast(w.E[[inv[int(t)] for t in tb]], "bf16"))
        ss = s[[inv[int(t)] for t in tb]].astype(np.float64)
        bound = (h[None, :] * (2.0 ** -4 * X + 2.0 ** -10 * ss[:, None])).sum(axis=1)
        bound += 2.0 ** -23 * (np.abs(lf) + np.abs(lb))
        assert np.all(np.abs(lf.astype(np.float64) - lb.astype(np.float64)) <= bound)


def test_masked_and_top_m_consistent():
    w = make_random(9, d=64, V=2048, Nc=32, dtype="bf16", rows=3)
    codes, s = f8.quantize_rows(w.E)
    M = f8.masked_logits_fp8(w.h, w.C, codes, s, w.offsets, w.tos, 3)
    tok, _ = f8.top_tokens_fp8(w.h, w.C, codes, s, w.offsets, w.tos, 3)
    tm, vm = f8.top_m_fp8(w.h, w.C, codes, s, w.offsets, w.tos, 3, 5)
    for b in range(3):
        row = M[b]
        assert tok[b] == int(np.flatnonzero(row == row.max()).min())
        assert tm[b, 0] == tok[b] and vm[b, 0] == row.max()
        fin = np.flatnonzero(np.isfinite(row))
        order = fin[np.lexsort((fin, -row[fin].astype(np.float64)))][:5]
        assert tm[b].tolist() == order.tolist()
