"""CPU oracle for the sparse head with FP8 embedding slabs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
product path never calls it and shares no code with it.

The pages gather the selected clusters' rows of the lm_head weight in the
model dtype (vLLM compare view "[Spec Decode] Add Gemma4 MTP speculative
decoding with centroids masking", ``Gemma4MTPMaskedEmbedder._select_and_score``).
Storing those rows as 8-bit floats halves the bytes the gather reads; the
pages do not do this (one of them names only a 4-bit target), so the format
is the OCP 8-bit floating point specification's E4M3 ("OFP8"): sign, four
exponent bits with bias 7, three mantissa bits, no infinities, S.1111.111 the
only NaN, largest finite 448, smallest normal 2^-6, subnormals k * 2^-9.

Definitions (readings of this module, also in the design notes):

* Each ordered-layout row j of E (bf16) gets a scale
  ``s_j = fl32(a_j / 448)`` with ``a_j = max_k |E[j,k]|`` (1.0 for an
  all-zero row) and codes ``q_jk = E4M3(fl64(E[j,k] / s_j))``: round to
  nearest, ties to even, magnitudes beyond 448 saturate to 448, the sign of
  zero kept.
* The logit of slot j for a bf16 row h is the canonical chain over the
  decoded codes, ``acc = sum_k h_k * dec(q_jk)`` in float64 sequentially
  from +0.0 (every product is exact), then ``L = fl32(fl64(acc * s_j))``
  with -0 turned into +0.
* Centroid scores, top-K and ties are those of the bf16 head (the centroids
  stay bf16); argmax, the masked row and the top-m use the logits above.
"""

from __future__ import annotations

import numpy as np

from .masked_head import candidate_slots, centroid_scores, topk_centroids, upcast

__all__ = ["e4m3_decode", "e4m3_encode", "quantize_rows", "fp8_chain_logits",
           "select_and_score_fp8", "top_tokens_fp8", "masked_logits_fp8", "top_m_fp8"]

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _rne_int(v: np.ndarray) -> np.ndarray:
    """Round float64 values (exact halves allowed) to the nearest integer,
    ties to even."""
    f = np.floor(v)
    r = v - f
    up = (r > 0.5) | ((r == 0.5) & (np.mod(f, 2) == 1))
    return f + up


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3 codes of float64 values: nearest, ties to even, saturating at
    +-448, sign of zero kept.  NaN is not accepted."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    out = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: multiples of 2^-9 below 2^-6 (rounding up to 8 * 2^-9
    # gives the smallest normal, whose code 0x08 follows 0x07)
    sub = a < 2.0 ** -6
    out[sub] = _rne_int(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        an = a[nrm]
        e = np.floor(np.log2(an)).astype(np.int64)
        # guard log2 rounding at exact powers of two
        e = np.where(np.exp2(e.astype(np.float64)) > an, e - 1, e)
        e = np.where(np.exp2((e + 1).astype(np.float64)) <= an, e + 1, e)
        mant = _rne_int(an / np.exp2(e.astype(np.float64)) * 8.0).astype(np.int64)   # 8 .. 16
        carry = mant == 16
        e = np.where(carry, e + 1, e)
        mant = np.where(carry, 8, mant)
        code = ((e + 7) << 3) | (mant - 8)
        code = np.where((e > 8) | ((e == 8) & (mant > 14)), 0x7E, code)   # saturate at 448
        out[nrm] = code
    return (out | sign).astype(np.uint8)


def quantize_rows(E_bits: np.ndarray):
    """``(codes [V,d] uint8, scales [V] float32)`` of bf16 rows (uint16 bits)."""
    X = upcast(E_bits, "bf16")
    a = np.abs(X).max(axis=1)
    s = np.where(a > 0, (a.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode(X / s.astype(np.float64)[:, None])
    return codes, s


def fp8_chain_logits(h_row: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 logits of one float64-valued hidden row against code rows:
    the sequential float64 chain over the decoded codes, times the row's
    scale in float64, rounded to fp32, plus 0.0."""
    Q = e4m3_decode(codes)                  # [n, d]
    acc = np.zeros(Q.shape[0], dtype=np.float64)
    for k in range(Q.shape[1]):
        acc = acc + h_row[k] * Q[:, k]      # exact product, one rounding per step
    L = (acc * scales.astype(np.float64)).astype(np.float32)
    return L + np.float32(0.0)


def select_and_score_fp8(h_row, C, codes, scales, offsets, tos, K: int):
    """(logits, token ids, selected centroids) of one bf16 row with FP8 slabs."""
    s = centroid_scores(np.atleast_2d(h_row), C, "bf16")[0]
    sel = topk_centroids(s[None, :], K)[0]
    slots = candidate_slots(sel, offsets)
    h64 = upcast(np.atleast_2d(h_row), "bf16")[0]
    logits = fp8_chain_logits(h64, codes[slots], scales[slots])
    return logits, np.asarray(tos)[slots].astype(np.int64), sel


def top_tokens_fp8(h, C, codes, scales, offsets, tos, K: int):
    """``[B]`` argmax tokens (ties to the lowest token, -1 without candidates)
    and the selected centroids ``[B, K]``."""
    h = np.atleast_2d(np.asarray(h))
    tok = np.full(h.shape[0], -1, dtype=np.int64)
    sels = []
    for b in range(h.shape[0]):
        logits, tokens, sel = select_and_score_fp8(h[b], C, codes, scales, offsets, tos, K)
        sels.append(sel)
        if len(logits):
            tok[b] = tokens[logits == logits.max()].min()
    return tok, np.array(sels, dtype=np.int64)


def masked_logits_fp8(h, C, codes, scales, offsets, tos, K: int):
    """``[B, V]`` fp32 rows: the FP8 logits at the candidate tokens, -inf
    elsewhere."""
    h = np.atleast_2d(np.asarray(h))
    V = len(tos)
    out = np.full((h.shape[0], V), -np.inf, dtype=np.float32)
    for b in range(h.shape[0]):
        logits, tokens, _ = select_and_score_fp8(h[b], C, codes, scales, offsets, tos, K)
        out[b, tokens] = logits
    return out


def top_m_fp8(h, C, codes, scales, offsets, tos, K: int, m: int):
    """The m best candidates per row by (logit desc, token asc), padded with
    (-1, -inf)."""
    h = np.atleast_2d(np.asarray(h))
    B = h.shape[0]
    tok = np.full((B, m), -1, dtype=np.int64)
    val = np.full((B, m), -np.inf, dtype=np.float32)
    for b in range(B):
        logits, tokens, _ = select_and_score_fp8(h[b], C, codes, scales, offsets, tos, K)
        order = np.lexsort((tokens, -logits.astype(np.float64)))[:m]
        tok[b, :len(order)] = tokens[order]
        val[b, :len(order)] = logits[order]
    return tok, val
