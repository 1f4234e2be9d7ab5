"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test targets a class of plausible oracle mistakes:

* hand-worked example (golden): wrong slot->token direction, wrong cluster
  lookup, wrong tie rule, -inf fill, sign of zero;
* exact rationals: a dropped or doubled term, a wrong sign, truncation instead
  of nearest-even rounding, summation in another order;
* numpy float64 matmul: a transposed operand, a wrong row of C or E;
* stable sort: top-K direction and tie order;
* dense lm_head brute force: masked rows equal the dense row on the candidates,
  K = Nc reduces the sparse argmax to the dense argmax.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import exact_dot, near_f32_midpoint, rne_f32, seq_error_bound
from workloads import f32_to_bf16_bits, make_random, make_workload, zipf_sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _as_f32(v):
    return np.float32(-np.inf) if v == "-inf" else np.float32(float(v))


# ---------------------------------------------------------------- golden example

def test_golden_scores_topk_tokens():
    g = _golden()
    C = np.array(g["centroids"], dtype=np.float32)
    E = np.array(g["emb_ordered"], dtype=np.float32)
    off = np.array(g["offsets"])
    tos = np.array(g["token_of_slot"])
    H = np.array([r["h"] for r in g["rows"]], dtype=np.float32)
    S = oracle.centroid_scores(H, C, "f32")
    for b, row in enumerate(g["rows"]):
        assert S[b].tolist() == row["scores"]
        for k, want in row["topk"].items():
            assert oracle.topk_centroids(S[b:b + 1], int(k))[0].tolist() == want
        for k, want in row["top_token"].items():
            tok, sel, _ = oracle.top_tokens(H[b:b + 1], C, E, off, tos, int(k), "f32")
            assert int(tok[0]) == want, (b, k)
            assert sel[0].tolist() == row["topk"][k]


def test_golden_masked_and_dense():
    g = _golden()
    C = np.array(g["centroids"], dtype=np.float32)
    E = np.array(g["emb_ordered"], dtype=np.float32)
    off = np.array(g["offsets"])
    tos = np.array(g["token_of_slot"])
    H = np.array([r["h"] for r in g["rows"]], dtype=np.float32)
    M, _ = oracle.masked_logits(H, C, E, off, tos, 2, "f32")
    D = oracle.dense_logits(H, E, tos, "f32")
    for b, row in enumerate(g["rows"]):
        want = np.array([_as_f32(v) for v in row["masked_K2"]], dtype=np.float32)
        assert M[b].view(np.uint32).tolist() == want.view(np.uint32).tolist(), b
        assert D[b].tolist() == row["dense"]
    # no -0 anywhere: all zero entries must carry a + sign
    assert not np.any(M.view(np.uint32) == 0x80000000)
    assert not np.any(D.view(np.uint32) == 0x80000000)


def test_golden_top_m():
    g = _golden()
    C = np.array(g["centroids"], dtype=np.float32)
    E = np.array(g["emb_ordered"], dtype=np.float32)
    off = np.array(g["offsets"])
    tos = np.array(g["token_of_slot"])
    for b, row in enumerate(g["rows"]):
        h = np.array([row["h"]], dtype=np.float32)
        for key, want in row["top_m"].items():
            if key == "derivation":
                continue
            K, m = int(key[1]), int(key.split("_m")[1])
            tok, val = oracle.top_m(h, C, E, off, tos, K, m, "f32")
            assert tok[0].tolist() == want["tokens"], (b, key)
            wv = np.array([_as_f32(v) for v in want["logits"]], dtype=np.float32)
            assert val[0].view(np.uint32).tolist() == wv.view(np.uint32).tolist(), (b, key)


def test_golden_rounding_cases():
    for case in _golden()["rounding_cases"]["cases"]:
        x = np.array(case["x"], dtype=np.float32)
        w = np.array(case["w"], dtype=np.float32)
        got = oracle.canonical_dots(x[None].astype(np.float64), w[None].astype(np.float64))[0, 0]
        assert got == np.float32(case["expect"]), case["why"]
        if case.get("expect_sign") == "+":
            assert got.view(np.uint32) == 0


# ---------------------------------------------------------------- exact rationals

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_canonical_dot_against_exact_rationals(dtype):
    rng = np.random.default_rng(11)
    n_mid = 0
    for trial in range(300):
        d = int(rng.integers(1, 17))
        x = rng.standard_normal(d).astype(np.float32) * np.float32(rng.choice([1e-3, 1, 1e3]))
        w = rng.standard_normal(d).astype(np.float32)
        if dtype == "bf16":
            xb, wb = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
            x64, w64 = oracle.upcast(xb, "bf16"), oracle.upcast(wb, "bf16")
        else:
            x64, w64 = x.astype(np.float64), w.astype(np.float64)
        q = exact_dot(x64, w64)
        got = oracle.canonical_dots(x64[None], w64[None])[0, 0]
        tol = seq_error_bound(x64, w64)
        # float64 sum of the exact products, to know whether it carries any error
        s = 0.0
        for a, b in zip(x64.tolist(), w64.tolist()):
            s = s + a * b
        assert abs(Fraction(s) - q) <= tol
        if Fraction(s) != q and near_f32_midpoint(q, tol):
            n_mid += 1
            continue
        assert got.view(np.uint32) == rne_f32(q).view(np.uint32), (trial, d)
    assert n_mid <= 3


def test_tiny_config_dense_sample_against_exact_rationals():
    w = make_workload("tiny")
    D = oracle.dense_logits(w.h[:2], w.E, w.tos, "f32")
    rng = np.random.default_rng(5)
    tok_of_slot = w.tos.astype(np.int64)
    for b in range(2):
        for j in rng.choice(w.V, size=64, replace=False):
            x = w.h[b].astype(np.float64)
            e = w.E[j].astype(np.float64)
            q = exact_dot(x, e)
            if near_f32_midpoint(q, seq_error_bound(x, e)):
                continue
            assert D[b, tok_of_slot[j]].view(np.uint32) == rne_f32(q).view(np.uint32)


def test_upcast_bf16_is_exact_widening():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 3.140625]
    got = oracle.upcast(bits, "bf16")
    assert got.tolist() == want
    assert np.signbit(got[3])


# ---------------------------------------------------------------- library routines

def test_canonical_dots_agree_with_float64_matmul():
    w = make_random(3, d=64, V=512, Nc=16, dtype="bf16", rows=8)
    X = oracle.upcast(w.h, "bf16")
    W = oracle.upcast(w.E, "bf16")
    got = oracle.canonical_dots(X, W)
    ref = (X @ W.T).astype(np.float32)
    ulp = np.abs(np.spacing(ref))
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
    assert np.mean(got == ref) > 0.999
    # a transposed or shifted operand would fail by far more than an ulp
    assert not np.allclose(oracle.canonical_dots(X, W[::-1]), ref)


def test_topk_equals_stable_argsort_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(50):
        Nc = int(rng.integers(2, 300))
        # few distinct values -> many ties; include both zeros
        S = rng.integers(-4, 5, size=(3, Nc)).astype(np.float32) * np.float32(0.5)
        S[S == 0] = np.where(rng.random((S == 0).sum()) < 0.5, -0.0, 0.0)
        K = int(rng.integers(1, Nc + 1))
        got = oracle.topk_centroids(S, K)
        for b in range(3):
            want = np.sort(np.argsort(-(S[b].astype(np.float64) + 0.0), kind="stable")[:K])
            assert got[b].tolist() == want.tolist()


def test_topk_definition_brute_force():
    rng = np.random.default_rng(8)
    for _ in range(40):
        Nc = int(rng.integers(1, 12))
        S = rng.integers(-2, 3, size=Nc).astype(np.float32)
        K = int(rng.integers(1, Nc + 1))
        sel = set(oracle.topk_centroids(S[None], K)[0].tolist())
        assert len(sel) == K
        for a in sel:
            for c in set(range(Nc)) - sel:
                # every kept centroid beats every dropped one under (score desc, id asc)
                assert S[a] > S[c] or (S[a] == S[c] and a < c)


def test_topk_nesting_and_zero_row():
    w = make_random(4, d=64, V=1024, Nc=64, dtype="bf16", rows=4)
    S = oracle.centroid_scores(w.h, w.C, "bf16")
    for K in range(1, 64):
        a = oracle.topk_centroids(S, K)
        b = oracle.topk_centroids(S, K + 1)
        for r in range(4):
            assert set(a[r]) <= set(b[r])
    zero = np.zeros((1, 64), dtype=np.uint16)
    Sz = oracle.centroid_scores(zero, w.C, "bf16")
    assert not np.any(Sz.view(np.uint32))          # every score is +0
    assert oracle.topk_centroids(Sz, 5)[0].tolist() == [0, 1, 2, 3, 4]


def test_duplicate_centroids_choose_lower_id():
    w = make_random(5, d=64, V=1024, Nc=32, dtype="bf16", rows=4)
    C = w.C.copy()
    S = oracle.centroid_scores(w.h, C, "bf16")
    best = int(np.argmax(S[0]))
    dup = 31 if best != 31 else 30
    C[dup] = C[best]
    S2 = oracle.centroid_scores(w.h, C, "bf16")
    assert S2[0, best] == S2[0, dup]
    sel = oracle.topk_centroids(S2[:1], 1)[0].tolist()
    assert sel == [min(best, dup)]


# ---------------------------------------------------------------- dense lm_head brute force

def _selected_tokens(sel, offsets, tos):
    out = set()
    for c in sel:
        out.update(tos[offsets[c]:offsets[c + 1]].tolist())
    return out


@pytest.mark.parametrize("case", ["tiny4", "tiny64", "ragged"])
def test_masked_equals_dense_on_candidates(case):
    if case.startswith("tiny"):
        w = make_workload("tiny")
        K = int(case[4:])
        h = w.h[:3]
    else:
        w = make_random(6, d=64, V=1000, Nc=40, dtype="bf16", rows=3, ragged=True)
        K = 7
        h = w.h
    M, sel = oracle.masked_logits(h, w.C, w.E, w.offsets, w.tos, K, w.dtype)
    D = oracle.dense_logits(h, w.E, w.tos, w.dtype)
    for b in range(h.shape[0]):
        toks = _selected_tokens(sel[b], w.offsets, w.tos)
        mask = np.zeros(w.V, dtype=bool)
        mask[list(toks)] = True
        assert np.array_equal(M[b, mask].view(np.uint32), D[b, mask].view(np.uint32))
        assert np.all(M[b, ~mask].view(np.uint32) == 0xFF800000)
        assert mask.sum() == int(sum(w.offsets[c + 1] - w.offsets[c] for c in sel[b]))


def test_full_K_gives_dense_argmax():
    for w, h in ((make_workload("tiny"), make_workload("tiny").h[:4]),
                 (make_random(7, d=64, V=600, Nc=30, dtype="bf16", rows=4, ragged=True), None)):
        h = w.h[:4] if h is None else h
        tok, sel, _ = oracle.top_tokens(h, w.C, w.E, w.offsets, w.tos, w.Nc, w.dtype)
        D = oracle.dense_logits(h, w.E, w.tos, w.dtype)
        assert tok.tolist() == np.argmax(D, axis=1).tolist()
        assert all(len(s) == w.Nc for s in sel)


def test_top_token_is_argmax_of_masked_row_and_monotone_in_K():
    w = make_random(8, d=64, V=2048, Nc=32, dtype="bf16", rows=6)
    prev = None
    for K in (1, 2, 4, 8, 16, 32):
        tok, _, best = oracle.top_tokens(w.h, w.C, w.E, w.offsets, w.tos, K, "bf16")
        M, _ = oracle.masked_logits(w.h, w.C, w.E, w.offsets, w.tos, K, "bf16")
        assert tok.tolist() == np.argmax(M, axis=1).tolist()
        assert best.tolist() == M.max(axis=1).tolist()
        if prev is not None:
            assert np.all(best >= prev)
        prev = best


def test_top_m_first_is_top_token_and_matches_masked_row():
    """top_m against get_top_tokens (m=1) and against a brute-force reading of
    the masked row: its finite entries ordered by (value desc, token asc)."""
    for w in (make_random(13, d=64, V=1024, Nc=32, dtype="bf16", rows=5),
              make_random(14, d=64, V=600, Nc=30, dtype="bf16", rows=4, ragged=True)):
        K, m = 3, 7
        tok1, _, best = oracle.top_tokens(w.h, w.C, w.E, w.offsets, w.tos, K, "bf16")
        t, v = oracle.top_m(w.h, w.C, w.E, w.offsets, w.tos, K, 1, "bf16")
        assert t[:, 0].tolist() == tok1.tolist()
        assert v[:, 0].tolist() == best.tolist()
        M, _ = oracle.masked_logits(w.h, w.C, w.E, w.offsets, w.tos, K, "bf16")
        t, v = oracle.top_m(w.h, w.C, w.E, w.offsets, w.tos, K, m, "bf16")
        for b in range(w.h.shape[0]):
            entries = sorted((-float(M[b, x]), x) for x in range(w.V) if np.isfinite(M[b, x]))
            want = [x for _, x in entries[:m]]
            want += [-1] * (m - len(want))
            assert t[b].tolist() == want, b
            for i, x in enumerate(want):
                if x < 0:
                    assert np.isneginf(v[b, i])
                else:
                    assert v[b, i].view(np.uint32) == M[b, x].view(np.uint32)


def test_top_m_ties_and_padding():
    # four equal candidates: ascending token order; m above the candidate
    # count pads with -1 / -inf
    d = 64
    h = np.zeros((1, d), dtype=np.float32)
    h[0, 0] = 1.0
    C = np.zeros((2, d), dtype=np.float32)
    C[0, 0] = 1.0
    E = np.zeros((8, d), dtype=np.float32)
    E[:4, 0] = 2.0
    off = np.array([0, 4, 8])
    tos = np.array([6, 1, 7, 3, 0, 2, 4, 5])
    tok, val = oracle.top_m(h, C, E, off, tos, 1, 6, "f32")
    assert tok[0].tolist() == [1, 3, 6, 7, -1, -1]
    assert val[0, :4].tolist() == [2.0] * 4 and np.all(np.isneginf(val[0, 4:]))


def test_tied_logits_choose_lowest_token():
    w = make_random(9, d=64, V=512, Nc=8, dtype="bf16", rows=2)
    tok, sel, _ = oracle.top_tokens(w.h[:1], w.C, w.E, w.offsets, w.tos, 2, "bf16")
    # copy the winner's embedding onto another candidate slot with a lower token id
    slots = np.concatenate([np.arange(w.offsets[c], w.offsets[c + 1]) for c in sel[0]])
    win = slots[w.tos[slots] == tok[0]][0]
    lower = [s for s in slots if w.tos[s] < tok[0]]
    if not lower:
        pytest.skip("winner already has the lowest candidate id")
    E = w.E.copy()
    E[lower[0]] = E[win]
    tok2, _, _ = oracle.top_tokens(w.h[:1], w.C, E, w.offsets, w.tos, 2, "bf16")
    assert tok2[0] == w.tos[lower[0]]


def test_empty_candidate_set_gives_minus_one():
    d = 64
    h = np.zeros((1, d), dtype=np.float32)
    h[0, 0] = 1.0
    C = np.zeros((4, d), dtype=np.float32)
    C[0, 0] = 5.0
    C[1, 0] = 4.0                               # clusters 0 and 1 win, both empty
    C[2, 0] = -1.0
    C[3, 0] = -2.0
    E = np.ones((8, d), dtype=np.float32)
    off = np.array([0, 0, 0, 4, 8])
    tos = np.arange(8)
    tok, sel, _ = oracle.top_tokens(h, C, E, off, tos, 2, "f32")
    assert sel[0].tolist() == [0, 1] and tok[0] == -1
    M, _ = oracle.masked_logits(h, C, E, off, tos, 2, "f32")
    assert np.all(np.isneginf(M))


def test_token_relabelling_is_equivariant():
    w = make_random(10, d=64, V=1024, Nc=16, dtype="bf16", rows=4)
    pi = np.random.default_rng(1).permutation(w.V)
    tos2 = pi[w.tos]
    tok, _, _ = oracle.top_tokens(w.h, w.C, w.E, w.offsets, w.tos, 3, "bf16")
    tok2, _, _ = oracle.top_tokens(w.h, w.C, w.E, w.offsets, tos2, 3, "bf16")
    M, _ = oracle.masked_logits(w.h, w.C, w.E, w.offsets, w.tos, 3, "bf16")
    M2, _ = oracle.masked_logits(w.h, w.C, w.E, w.offsets, tos2, 3, "bf16")
    assert tok2.tolist() == pi[tok].tolist()
    assert np.array_equal(M2[:, pi].view(np.uint32), M.view(np.uint32))


def test_rows_are_independent_of_batch():
    w = make_random(12, d=64, V=1024, Nc=32, dtype="bf16", rows=8)
    tok8, sel8, _ = oracle.top_tokens(w.h, w.C, w.E, w.offsets, w.tos, 4, "bf16")
    tok3, sel3, _ = oracle.top_tokens(w.h[:3], w.C, w.E, w.offsets, w.tos, 4, "bf16")
    assert tok8[:3].tolist() == tok3.tolist()
    assert sel8[:3].tolist() == sel3.tolist()


# ---------------------------------------------------------------- synthetic inputs

def test_zipf_sizes_skewed_config():
    sizes = zipf_sizes(2048, 262144, 1.1, np.arange(2048))
    assert sizes.sum() == 262144
    assert sizes.max() == 44286 and sizes.min() == 10
    assert np.all(np.diff(sizes) <= 0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -1.5], dtype=np.float32)
    got = f32_to_bf16_bits(x).tolist()
    assert got == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBFC0]


def test_exact_helpers_selfcheck():
    assert rne_f32(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert rne_f32(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1 + 2 ** -22)
