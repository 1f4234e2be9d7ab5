"""CPU oracle for the centroid-masked sparse LM head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
product path (the HIP library and its Python binding) never calls it and
shares no code with it.

What it computes follows the vLLM compare view "[Spec Decode] Add Gemma4 MTP
speculative decoding with centroids masking", diff of ``gemma4_mtp.py``, class
``Gemma4MTPMaskedEmbedder``:

* ``_select_and_score``: centroid projection of each hidden row, top-K over
  the centroid scores, lookup of the token ids owned by the selected
  centroids through ``token_ordering`` viewed as ``[num_centroids,
  vocab_size_per_centroid]``, gather of those rows of the lm_head weight and
  their dot products with the hidden row;
* ``forward``: a full-vocabulary row holding those scores at the selected
  token ids and the fill value everywhere else;
* ``get_top_tokens``: the token id of the largest sparse score.

Readings where the page leaves a step open (each is also listed with its
reason in the design notes):

* Dot products use one canonical rounding (the "canonical key"): every
  element is widened exactly to float64, the sum runs sequentially over the
  hidden dimension from +0.0, ``s <- fl64(s + x_k * w_k)`` (each product is
  exact in float64 for fp32 and bf16 inputs), and the result is rounded to
  fp32 nearest-even, then ``+0.0`` turns a -0 into +0.  The page uses the
  model dtype and leaves order and precision to the library.
* Top-K ties go to the lowest centroid id, argmax ties to the lowest token id;
  the top-K result is a set, reported in ascending id order.
* The fill value of ``forward`` is -inf in fp32 (the docstring's reading) and
  the logits are fp32, not the model dtype.
* ``token_ordering`` is read as slot -> token id (how the code uses it), and
  the equal-size cluster view generalises to cluster offsets: cluster c owns
  slots ``[offsets[c], offsets[c+1])``.  Equal clusters are
  ``offsets[c] = c * V // Nc``.

Inputs: ``h [B,d]``, ``C [Nc,d]``, ``E [V,d]`` (ordered layout: row j is the
embedding of token ``tos[j]``), ``offsets [Nc+1]``, ``tos [V]``; element type
``"f32"`` (float32 arrays) or ``"bf16"`` (uint16 bit patterns).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "upcast",
    "canonical_dots",
    "centroid_scores",
    "topk_centroids",
    "candidate_slots",
    "select_and_score",
    "masked_logits",
    "top_tokens",
    "top_m",
    "log_softmax_candidates",
    "top_m_log_softmax",
    "dense_logits",
]


def upcast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp32 values or bf16 bit patterns to float64 exactly."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(
            np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown element type {dtype!r}")


def canonical_dots(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Canonical dot products of every row of X with every row of W.

    ``X [n,d]`` and ``W [m,d]`` are float64 holding fp32- or bf16-valued
    elements.  Entry (i, j) is ``s_d`` rounded to fp32, plus 0.0, where
    ``s_0 = +0.0`` and ``s_{k+1} = fl64(s_k + X[i,k] * W[j,k])``.  The loop
    runs over k in order; each step is vectorised over the n*m independent
    sums, which leaves every individual sum untouched.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    n, d = X.shape
    m, d2 = W.shape
    if d != d2:
        raise ValueError("hidden sizes differ")
    WT = np.ascontiguousarray(W.T)
    s = np.zeros((n, m), dtype=np.float64)
    for k in range(d):
        s += X[:, k:k + 1] * WT[k][None, :]
    out = s.astype(np.float32)
    out += np.float32(0.0)
    return out


def centroid_scores(h: np.ndarray, C: np.ndarray, dtype: str) -> np.ndarray:
    """Scores of every hidden row against every centroid: ``[B, Nc]`` fp32.

    The centroid projection ``self.centroids(hidden_states)`` of
    ``_select_and_score`` (a bias-free linear layer), in canonical rounding.
    """
    return canonical_dots(upcast(h, dtype), upcast(C, dtype))


def topk_centroids(S: np.ndarray, K: int) -> np.ndarray:
    """The K best centroids of each row of ``S [B, Nc]``: ``[B, K]`` ascending.

    ``torch.topk(..., k=K)`` of ``_select_and_score`` with a fixed tie rule:
    centroids are ranked by (score descending, id ascending) and the first K
    are kept; -0 and +0 are equal scores.
    """
    S = np.atleast_2d(np.asarray(S, dtype=np.float32))
    B, Nc = S.shape
    if not 1 <= K <= Nc:
        raise ValueError("K must lie in [1, Nc]")
    ids = np.arange(Nc)
    out = np.empty((B, K), dtype=np.int64)
    for b in range(B):
        key = -(S[b].astype(np.float64) + 0.0)
        order = np.lexsort((ids, key))      # last key is primary
        out[b] = np.sort(order[:K])
    return out


def candidate_slots(selected: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Slots owned by the selected centroids, in the order the ids are given.

    ``clusters[top_k_indices]`` of ``_select_and_score`` with the cluster view
    generalised to offsets.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    parts = [np.arange(offsets[c], offsets[c + 1]) for c in selected]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def select_and_score(h_row, C, E, offsets, tos, K: int, dtype: str):
    """One row of ``_select_and_score``.

    Returns ``(logits fp32 [n], token_ids int64 [n], selected ascending [K])``:
    the canonical dot products of the hidden row with the embeddings of every
    token owned by the K selected centroids, and those tokens' ids.
    """
    h64 = upcast(np.asarray(h_row)[None, :], dtype)
    S = canonical_dots(h64, upcast(C, dtype))
    sel = topk_centroids(S, K)[0]
    slots = candidate_slots(sel, offsets)
    logits = canonical_dots(h64, upcast(np.asarray(E)[slots], dtype))[0]
    tokens = np.asarray(tos, dtype=np.int64)[slots]
    return logits, tokens, sel


def masked_logits(h, C, E, offsets, tos, K: int, dtype: str):
    """``forward``: ``[B, V]`` fp32 rows, scores at candidate tokens, -inf elsewhere.

    Also returns the selected centroids ``[B, K]``.
    """
    h = np.atleast_2d(np.asarray(h))
    V = len(tos)
    out = np.full((h.shape[0], V), -np.inf, dtype=np.float32)
    sels = []
    for b in range(h.shape[0]):
        logits, tokens, sel = select_and_score(h[b], C, E, offsets, tos, K, dtype)
        out[b, tokens] = logits
        sels.append(sel)
    return out, np.array(sels, dtype=np.int64)


def top_tokens(h, C, E, offsets, tos, K: int, dtype: str):
    """``get_top_tokens``: ``[B]`` token ids of the largest sparse score.

    Ties go to the lowest token id; a row whose selected centroids own no
    token at all gives -1.  Also returns the selected centroids ``[B, K]``
    and the maximum score of each row (NaN for an empty row).
    """
    h = np.atleast_2d(np.asarray(h))
    B = h.shape[0]
    tok = np.full(B, -1, dtype=np.int64)
    best = np.full(B, np.nan, dtype=np.float32)
    sels = []
    for b in range(B):
        logits, tokens, sel = select_and_score(h[b], C, E, offsets, tos, K, dtype)
        sels.append(sel)
        if len(logits):
            m = logits.max()
            tok[b] = tokens[logits == m].min()
            best[b] = m
    return tok, np.array(sels, dtype=np.int64), best


def top_m(h, C, E, offsets, tos, K: int, m: int, dtype: str):
    """The m best candidates of each row: ``[B, m]`` token ids and their fp32
    logits, ordered by (logit descending, token ascending).

    The next step after ``get_top_tokens`` for tree drafting or sampling: the
    same candidates as the masked row, reduced to its m largest entries
    without building the row.  A row with fewer than m candidates is padded
    with token -1 and logit -inf.
    """
    h = np.atleast_2d(np.asarray(h))
    B = h.shape[0]
    tok = np.full((B, m), -1, dtype=np.int64)
    val = np.full((B, m), -np.inf, dtype=np.float32)
    for b in range(B):
        logits, tokens, _ = select_and_score(h[b], C, E, offsets, tos, K, dtype)
        order = np.lexsort((tokens, -logits.astype(np.float64)))[:m]
        tok[b, :len(order)] = tokens[order]
        val[b, :len(order)] = logits[order]
    return tok, val


def log_softmax_candidates(logits) -> np.ndarray:
    """Log-probabilities of a row's candidates under a softmax over the
    candidate set alone: ``log p_i = l_i - log(sum_c exp(l_c))``.

    This is the softmax a sampler takes over ``forward``'s masked row, whose
    -inf entries contribute exp(-inf) = 0 (same page, class
    ``Gemma4MTPMaskedEmbedder``, ``forward``).  The page fixes no precision:
    in float64, with ``M`` the largest logit and ``T = sum_c exp(l_c - M)``
    over every candidate but one that holds ``M``, ``log p_i = (l_i - M) -
    log1p(T)``.  The shift keeps every exponential at most 1; subtracting
    from the shifted logit (rather than adding ``M`` back first), and
    log1p(T) rather than log(1 + T), keep the relative precision of
    log-probabilities near 0, where the largest candidate dominates.  Each
    result is rounded once to fp32 (nearest-even).  An empty row gives an
    empty result.
    """
    x = np.asarray(logits, dtype=np.float64).ravel()
    if x.size == 0:
        return np.zeros(0, dtype=np.float32)
    top = int(np.argmax(x))
    sh = x - x[top]
    t = np.sum(np.exp(np.delete(sh, top)))
    return (sh - np.log1p(t)).astype(np.float32)


def top_m_log_softmax(h, C, E, offsets, tos, K: int, m: int, dtype: str):
    """``top_m``'s tokens with their log-probabilities under the softmax over
    each row's candidate set (``log_softmax_candidates``) instead of their
    logits: ``[B, m]`` token ids (ordered as in ``top_m``) and fp32
    log-probabilities, padded with token -1 and -inf."""
    h = np.atleast_2d(np.asarray(h))
    B = h.shape[0]
    tok = np.full((B, m), -1, dtype=np.int64)
    val = np.full((B, m), -np.inf, dtype=np.float32)
    for b in range(B):
        logits, tokens, _ = select_and_score(h[b], C, E, offsets, tos, K, dtype)
        lp = log_softmax_candidates(logits)
        order = np.lexsort((tokens, -logits.astype(np.float64)))[:m]
        tok[b, :len(order)] = tokens[order]
        val[b, :len(order)] = lp[order]
    return tok, val


def dense_logits(h, E, tos, dtype: str, chunk: int = 8192) -> np.ndarray:
    """Dense lm_head logits ``[B, V]`` in canonical rounding, indexed by token id.

    The plain (unmasked) head: every token's embedding dotted with every row.
    ``E`` is in the ordered layout, so token ``tos[j]`` takes row j.  Work is
    split over groups of slots only to bound memory.
    """
    h64 = upcast(np.atleast_2d(np.asarray(h)), dtype)
    V = len(tos)
    tos = np.asarray(tos, dtype=np.int64)
    out = np.empty((h64.shape[0], V), dtype=np.float32)
    for j0 in range(0, V, chunk):
        j1 = min(V, j0 + chunk)
        out[:, tos[j0:j1]] = canonical_dots(h64, upcast(np.asarray(E)[j0:j1], dtype))
    return out
