"""CPU oracle for the fused draft step around the sparse head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
product path never calls it and shares no code with it.

In the vLLM compare view "[Spec Decode] Add Gemma4 MTP speculative decoding
with centroids masking" (diff of ``gemma4_mtp.py``), one draft step of the
multi-token predictor ends with the final ``RMSNorm`` (``self.norm``,
``RMSNorm(hidden_size, eps=rms_norm_eps)``, class ``Gemma4MultiTokenPredictor``,
``forward``): its output is the draft hidden state that the masked head
scores, and the next step starts from ``embed_input_ids``, the backbone
embedding of the chosen token times ``normalizer`` (the square root of the
backbone hidden size, a float32 buffer).  This module composes

    x --RMSNorm--> h --sparse head (argmax)--> token --embed * normalizer--> e

Readings where the page leaves a step open (also listed in the design notes):

* RMSNorm is the plain one: ``y_k = x_k * w_k / sqrt(mean_j x_j^2 + eps)``.
  Its canonical rounding ("canonical norm"): the sum of squares is the same
  sequential float64 chain as every dot product of the head, applied to x
  with itself: ``ss_0 = +0.0``, ``ss_{k+1} = fl64(ss_k + x_k * x_k)`` for
  k = 0 .. d-1 in order (each square is exact in float64), kept in float64;
  then ``v = ss / d + eps`` (eps widened from float32), ``r = 1 / sqrt(v)``,
  ``y_k = (x_k * r) * w_k``, every step one correctly rounded float64
  operation; ``y`` is rounded to float32 (nearest-even) and, for bf16 heads,
  that float32 to bf16 (nearest-even).
* The embedding product follows the model's dtype rule: the bf16 (or fp32)
  table element times the float32 ``normalizer`` in float32 (one rounding),
  then, for bf16, rounded to bf16 (nearest-even).  A row with no candidate
  (token -1) gets an all-zero embedding.
"""

from __future__ import annotations

import numpy as np

from .masked_head import top_tokens, upcast

__all__ = ["f32_to_bf16_bits", "sum_of_squares", "rms_norm", "embed_rows", "draft_step"]

CHUNK = 64


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits.

    NaN becomes the quiet NaN 0x7FC0 (sign kept); everything else, infinities
    included, follows the usual carry into the exponent.
    """
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    out = np.where(nan, ((u >> 16) & 0x8000) | 0x7FC0, rounded)
    return out.astype(np.uint16)


def sum_of_squares(x: np.ndarray, dtype: str) -> np.ndarray:
    """Float64 sum of squares of each row of x ``[B,d]``, the canonical
    chain: from +0.0, one square (exact in float64) added per step in
    hidden-dimension order, one rounding per step, no final rounding."""
    X = upcast(x, dtype)
    ss = np.zeros(X.shape[0], dtype=np.float64)   # +0.0
    for k in range(X.shape[1]):                   # hidden-dimension order
        ss = ss + X[:, k] * X[:, k]
    return ss


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float, dtype: str) -> np.ndarray:
    """Canonical RMSNorm of the rows of x ``[B,d]`` with weight w ``[d]``.

    Returns bf16 bit patterns (``uint16``) for ``dtype="bf16"``, float32
    values for ``"f32"``.  d must be a multiple of 64.
    """
    X = upcast(x, dtype)
    W = upcast(w, dtype)
    n, d = X.shape
    if d % CHUNK:
        raise ValueError("d must be a multiple of 64")
    ss = sum_of_squares(x, dtype)
    v = ss / np.float64(d) + np.float64(np.float32(eps))
    r = np.float64(1.0) / np.sqrt(v)
    y = (X * r[:, None]) * W[None, :]
    y32 = y.astype(np.float32)
    return f32_to_bf16_bits(y32) if dtype == "bf16" else y32


def embed_rows(table: np.ndarray, tokens: np.ndarray, normalizer: float, dtype: str) -> np.ndarray:
    """``table[tok] * normalizer`` per token (float32 product, then the head
    dtype); all zeros for token -1."""
    tok = np.asarray(tokens)
    emb_dim = table.shape[1]
    n32 = np.float32(normalizer)
    out = np.zeros((len(tok), emb_dim), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b, t in enumerate(tok):
        if t < 0:
            continue
        e = upcast(table[t], dtype).astype(np.float32)   # exact
        p = e * n32                                      # one float32 rounding
        out[b] = f32_to_bf16_bits(p) if dtype == "bf16" else p
    return out


def draft_step(x, w, eps, C, E, offsets, tos, K, table, normalizer, dtype):
    """(h, tokens, embeddings, selected): the normalised rows, their top
    tokens under the sparse head, the scaled embeddings of those tokens
    (``None`` without a table) and the selected centroids ``[B, K]``."""
    h = rms_norm(x, w, eps, dtype)
    tokens, sel, _ = top_tokens(h, C, E, offsets, tos, K, dtype)
    emb = None if table is None else embed_rows(table, tokens, normalizer, dtype)
    return h, tokens, emb, sel
