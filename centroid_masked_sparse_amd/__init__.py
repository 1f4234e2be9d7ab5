"""Centroid-masked sparse LM head for MI355X (gfx950).

A thin Python binding over the C ABI of ``include/ce.h`` (``libce.so``).  It
only marshals arguments: torch supplies device memory and streams, and every
step of the computation runs in the library's HIP kernels.  If the library is
missing, every call raises; there is no fallback implementation.

The head is the one of Gemma4MTPMaskedEmbedder in the vLLM compare view
"[Spec Decode] Add Gemma4 MTP speculative decoding with centroids masking"
(diff of gemma4_mtp.py): ``top_tokens`` is get_top_tokens, ``masked_logits``
is forward, and ``score_centroids`` / ``topk`` expose the first two steps of
_select_and_score.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import _ffi
from ._ffi import (CE_BF16, CE_F32, CE_MAX_TOP_M, CE_OP_DRAFT_STEP, CE_OP_MASKED_LOGITS,
                   CE_OP_SCORE, CE_OP_TOP_M, CE_OP_TOP_M_LOG_SOFTMAX, CE_OP_TOP_TOKENS, CE_OP_TOPK,
                   CeError, check)

__all__ = ["Head", "Graph", "CeError", "load_library"]


def load_library():
    """Load ``libce.so`` (raises when it has not been built)."""
    return _ffi.load()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CE_BF16
    if t.dtype == torch.float32:
        return CE_F32
    raise TypeError(f"unsupported element type {t.dtype}; use float32 or bfloat16")


def _stream_handle(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _host_i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


class Graph:
    """An instantiated HIP graph of one captured call."""

    def __init__(self, lib, handle, keep):
        self._lib = lib
        self._handle = handle
        self._keep = keep

    def launch(self, stream=None) -> None:
        s = stream if stream is not None else _stream_handle(self._keep[0].device)
        check(self._lib.ce_graph_launch(self._handle, s), "ce_graph_launch")

    def close(self) -> None:
        if self._handle:
            self._lib.ce_graph_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Head:
    """One prepared head: centroids ``[Nc, d]``, ordered embeddings ``[V, d]``.

    ``token_of_slot`` (host, ``[V]``) gives the token id of each embedding row;
    ``cluster_offsets`` (host, ``[Nc+1]``) gives each centroid's slot range, or
    None for equal clusters.  ``max_B``/``max_K`` bound later calls.
    ``slabs="fp8"`` stores the embedding slabs as OCP E4M3 codes with a
    float32 scale per row (bf16 heads only; logits change accordingly).

    Calls run on torch's current stream and share one cached workspace per
    op, so calls of the same op issued on different streams at once would
    overwrite each other's scratch: keep one head per stream, or pass each
    stream's own workspace through the C ABI (``new_workspace``).
    """

    _PROJ = {"auto": _ffi.CE_PROJ_AUTO, "exact": _ffi.CE_PROJ_EXACT, "mfma": _ffi.CE_PROJ_MFMA}

    def __init__(self, centroids, emb_ordered, token_of_slot, cluster_offsets=None,
                 max_B: int = 64, max_K: int | None = None, slabs: str = "native",
                 projection: str = "auto"):
        if slabs not in ("native", "fp8"):
            raise ValueError("slabs must be 'native' or 'fp8'")
        if projection not in self._PROJ:
            raise ValueError("projection must be 'auto', 'exact' or 'mfma'")
        torch = _torch()
        self._lib = _ffi.load()
        for name, t in (("centroids", centroids), ("emb_ordered", emb_ordered)):
            if not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
                raise ValueError(f"{name} must be a contiguous 2-D GPU tensor")
        if centroids.dtype != emb_ordered.dtype:
            raise TypeError("centroids and emb_ordered must share one element type")
        self.device = centroids.device
        self.Nc, self.d = centroids.shape
        self.V = emb_ordered.shape[0]
        self.dtype = centroids.dtype
        self.max_B = int(max_B)
        self.max_K = int(max_K if max_K is not None else self.Nc)
        self._tos = _host_i32(token_of_slot)
        self._off = None if cluster_offsets is None else _host_i32(cluster_offsets)
        self._keep = (centroids, emb_ordered)
        desc = _ffi.HeadDesc(
            d=self.d, V=self.V, Nc=self.Nc, max_B=self.max_B, max_K=self.max_K,
            dtype=_dtype_code(centroids), centroids=centroids.data_ptr(),
            emb_ordered=emb_ordered.data_ptr(),
            cluster_offsets=None if self._off is None else
            self._off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            token_of_slot=self._tos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            slab_format=_ffi.CE_SLAB_FP8_E4M3 if slabs == "fp8" else _ffi.CE_SLAB_NATIVE,
            projection=self._PROJ[projection])
        self.slabs = slabs
        handle = ctypes.c_void_p()
        check(self._lib.ce_head_create(ctypes.byref(desc), ctypes.byref(handle)), "ce_head_create")
        self._handle = handle
        nbytes = ctypes.c_size_t()
        check(self._lib.ce_head_persistent_bytes(handle, ctypes.byref(nbytes)),
              "ce_head_persistent_bytes")
        self._persist = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=self.device)
        check(self._lib.ce_head_prepare(handle, self._persist.data_ptr(), nbytes.value,
                                        _stream_handle(self.device)), "ce_head_prepare")
        self._ws = {}

    # ------------------------------------------------------------------ helpers
    def workspace_bytes(self, B: int, K: int, op: int) -> int:
        n = ctypes.c_size_t()
        check(self._lib.ce_workspace_bytes(self._handle, B, K, op, ctypes.byref(n)),
              "ce_workspace_bytes")
        return n.value

    def new_workspace(self, B: int, K: int, op: int):
        torch = _torch()
        return torch.empty(max(self.workspace_bytes(B, K, op), 256), dtype=torch.uint8,
                           device=self.device)

    def _workspace(self, B: int, K: int, op: int):
        need = self.workspace_bytes(B, K, op)
        ws = self._ws.get(op)
        if ws is None or ws.numel() < need:
            ws = self.new_workspace(B, K, op)
            self._ws[op] = ws
        return ws

    def _check_h(self, h):
        if not h.is_cuda or h.device != self.device or h.dtype != self.dtype:
            raise ValueError("h must be on the head's device with the head's element type")
        if h.dim() != 2 or h.shape[1] != self.d or not h.is_contiguous():
            raise ValueError(f"h must be a contiguous [B, {self.d}] tensor")
        return h.shape[0]

    def _k(self, K):
        return self.max_K if K is None else int(K)

    def repair_counts(self) -> tuple[int, int]:
        """(rows whose top-K boundary took recomputed canonical keys, rows
        recomputed whole) since prepare, for the MFMA projection.  Synchronises."""
        c = (ctypes.c_uint64 * 2)()
        check(self._lib.ce_head_repair_counts(self._handle, c), "ce_head_repair_counts")
        return int(c[0]), int(c[1])

    def approx_scores(self, h, out=None):
        """``[B, Nc]`` fp32 scores of the MFMA projection alone (bf16 heads), the
        approximate values the certified top-K starts from."""
        torch = _torch()
        B = self._check_h(h)
        if out is None:
            out = torch.empty((B, self.Nc), dtype=torch.float32, device=self.device)
        check(self._lib.ce_probe_approx_scores(self._handle, h.data_ptr(), B, out.data_ptr(),
                                               _stream_handle(self.device)), "ce_probe_approx_scores")
        return out

    # ------------------------------------------------------------------ calls
    def score_centroids(self, h, out=None):
        """``[B, Nc]`` fp32 canonical scores of every row against every centroid."""
        torch = _torch()
        B = self._check_h(h)
        if out is None:
            out = torch.empty((B, self.Nc), dtype=torch.float32, device=self.device)
        check(self._lib.ce_score_centroids(self._handle, h.data_ptr(), B, out.data_ptr(),
                                           _stream_handle(self.device)), "ce_score_centroids")
        return out

    def topk(self, scores, K: int, out=None):
        """``[B, K]`` int32 ascending ids of the K best centroids of each row."""
        torch = _torch()
        if scores.dtype != torch.float32 or scores.dim() != 2 or scores.shape[1] != self.Nc \
                or not scores.is_contiguous() or scores.device != self.device:
            raise ValueError(f"scores must be a contiguous fp32 [B, {self.Nc}] tensor on the device")
        B = scores.shape[0]
        if out is None:
            out = torch.empty((B, K), dtype=torch.int32, device=self.device)
        check(self._lib.ce_topk(self._handle, scores.data_ptr(), B, K, out.data_ptr(),
                                _stream_handle(self.device)), "ce_topk")
        return out

    def top_tokens(self, h, K: int | None = None, out=None, topk_out=None):
        """``[B]`` int32 greedy token ids (get_top_tokens)."""
        torch = _torch()
        B = self._check_h(h)
        K = self._k(K)
        if out is None:
            out = torch.empty((B,), dtype=torch.int32, device=self.device)
        ws = self._workspace(B, K, CE_OP_TOP_TOKENS)
        check(self._lib.ce_top_tokens(self._handle, h.data_ptr(), B, K, out.data_ptr(),
                                      0 if topk_out is None else topk_out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream_handle(self.device)),
              "ce_top_tokens")
        return out

    def top_tokens_static(self, h, K: int | None = None, out=None, topk_out=None):
        """``top_tokens`` through ``ce_top_tokens_static``: no workspace is
        allocated (the library's static per-GPU scratch is used), so calls on
        one GPU must not overlap."""
        torch = _torch()
        B = self._check_h(h)
        K = self._k(K)
        if out is None:
            out = torch.empty((B,), dtype=torch.int32, device=self.device)
        check(self._lib.ce_top_tokens_static(self._handle, h.data_ptr(), B, K, out.data_ptr(),
                                             0 if topk_out is None else topk_out.data_ptr(),
                                             _stream_handle(self.device)), "ce_top_tokens_static")
        return out

    def masked_logits(self, h, K: int | None = None, out=None, topk_out=None):
        """``[B, V]`` fp32 logits, -inf outside the candidates (forward)."""
        torch = _torch()
        B = self._check_h(h)
        K = self._k(K)
        if out is None:
            out = torch.empty((B, self.V), dtype=torch.float32, device=self.device)
        ws = self._workspace(B, K, CE_OP_MASKED_LOGITS)
        check(self._lib.ce_masked_logits(self._handle, h.data_ptr(), B, K, out.data_ptr(),
                                         0 if topk_out is None else topk_out.data_ptr(),
                                         ws.data_ptr(), ws.numel(), _stream_handle(self.device)),
              "ce_masked_logits")
        return out

    def top_m(self, h, m: int, K: int | None = None, out=None, logits_out=None, topk_out=None,
              log_softmax: bool = False):
        """The m best candidates per row: ``([B, m]`` int32 token ids, ``[B, m]``
        fp32 logits), ordered by logit descending then token id ascending;
        rows with fewer than m candidates are padded with -1 / -inf.  With
        ``log_softmax`` the second output holds each candidate's
        log-probability under the softmax over the row's candidates
        (``ce_top_m_log_softmax``) instead of its logit."""
        torch = _torch()
        B = self._check_h(h)
        K = self._k(K)
        if out is None:
            out = torch.empty((B, m), dtype=torch.int32, device=self.device)
        if logits_out is None:
            logits_out = torch.empty((B, m), dtype=torch.float32, device=self.device)
        op = CE_OP_TOP_M_LOG_SOFTMAX if log_softmax else CE_OP_TOP_M
        name = "ce_top_m_log_softmax" if log_softmax else "ce_top_m"
        ws = self._workspace(B, K, op)
        check(getattr(self._lib, name)(self._handle, h.data_ptr(), B, K, m, out.data_ptr(),
                                       logits_out.data_ptr(),
                                       0 if topk_out is None else topk_out.data_ptr(),
                                       ws.data_ptr(), ws.numel(), _stream_handle(self.device)),
              name)
        return out, logits_out

    def draft_step(self, x, norm_weight, eps: float, K: int | None = None, emb_table=None,
                   normalizer: float = 1.0, h_out=None, out=None, emb_out=None, topk_out=None):
        """One fused draft step: the final RMSNorm of the rows x, the top token of
        each normalised row, and (given ``emb_table``, ``[V, emb_dim]`` indexed
        by token id) that token's embedding times ``normalizer``.

        Returns ``(h, tokens, emb)`` (``emb`` is None without a table)."""
        torch = _torch()
        B = self._check_h(x)
        K = self._k(K)
        if norm_weight.dtype != self.dtype or not norm_weight.is_cuda or norm_weight.numel() != self.d:
            raise ValueError("norm_weight must be a [d] tensor of the head's dtype on its device")
        if h_out is None:
            h_out = torch.empty_like(x)
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=self.device)
        emb_dim = 0
        if emb_table is not None:
            if emb_table.dtype != self.dtype or emb_table.dim() != 2 or not emb_table.is_contiguous():
                raise ValueError("emb_table must be a contiguous [V, emb_dim] tensor of the head's dtype")
            emb_dim = emb_table.shape[1]
            if emb_out is None:
                emb_out = torch.empty((B, emb_dim), dtype=self.dtype, device=self.device)
        ws = self._workspace(B, K, CE_OP_DRAFT_STEP)
        check(self._lib.ce_draft_step(self._handle, x.data_ptr(), norm_weight.data_ptr(), float(eps),
                                      B, K, h_out.data_ptr(), out.data_ptr(),
                                      0 if emb_table is None else emb_table.data_ptr(), emb_dim,
                                      float(normalizer),
                                      0 if emb_out is None else emb_out.data_ptr(),
                                      0 if topk_out is None else topk_out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream_handle(self.device)),
              "ce_draft_step")
        return h_out, out, (emb_out if emb_table is not None else None)

    def capture(self, op: int, h, K: int | None, out, topk_out=None, stream=None, *, m: int = 0,
                logits_out=None, norm_weight=None, eps: float = 0.0, h_out=None, emb_table=None,
                normalizer: float = 1.0, emb_out=None) -> Graph:
        """Capture one call of any op into a HIP graph (with its own workspace).

        ``op`` is one of the ``OP_*`` codes; ``h`` is the op's input (the rows,
        the ``[B, Nc]`` scores for ``OP_TOPK``, the rows before the norm for
        ``OP_DRAFT_STEP``) and ``out`` its first output (scores, top-K ids,
        tokens or logits).  ``OP_TOP_M`` and ``OP_TOP_M_LOG_SOFTMAX`` also take
        ``m`` and ``logits_out``;
        ``OP_DRAFT_STEP`` takes ``norm_weight``, ``eps``, ``h_out`` and
        optionally ``emb_table``, ``normalizer`` and ``emb_out``.  Every tensor
        is read or written at the same address on every launch.  ``stream``
        (a torch stream, not the null stream) is used for capture.
        """
        torch = _torch()
        B = h.shape[0]
        if op == CE_OP_TOPK:
            if h.dtype != torch.float32 or h.dim() != 2 or h.shape[1] != self.Nc or not h.is_contiguous():
                raise ValueError(f"scores must be a contiguous fp32 [B, {self.Nc}] tensor")
        else:
            self._check_h(h)
        K = 1 if op == CE_OP_SCORE else self._k(K)
        ws = self.new_workspace(B, K, op) if op not in (CE_OP_SCORE, CE_OP_TOPK) else None
        ptr = (lambda t: 0 if t is None else t.data_ptr())
        call = _ffi.CeCall(
            op=op, in_=h.data_ptr(), B=B, K=K, m=int(m), out=out.data_ptr(),
            out_logits=ptr(logits_out), topk_ids=ptr(topk_out), ws=ptr(ws),
            ws_bytes=0 if ws is None else ws.numel(), norm_weight=ptr(norm_weight),
            eps=float(eps), h_out=ptr(h_out), emb_table=ptr(emb_table),
            emb_dim=0 if emb_table is None else int(emb_table.shape[1]),
            normalizer=float(normalizer), emb_out=ptr(emb_out))
        s = stream if stream is not None else torch.cuda.Stream(self.device)
        g = ctypes.c_void_p()
        check(self._lib.ce_graph_capture_call(self._handle, ctypes.byref(call), s.cuda_stream,
                                              ctypes.byref(g)), "ce_graph_capture_call")
        keep = (h, out, topk_out, ws, logits_out, norm_weight, h_out, emb_table, emb_out, self)
        return Graph(self._lib, g, keep)

    def close(self) -> None:
        if getattr(self, "_handle", None):
            self._lib.ce_head_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


OP_SCORE = CE_OP_SCORE
OP_TOPK = CE_OP_TOPK
OP_TOP_TOKENS = CE_OP_TOP_TOKENS
OP_MASKED_LOGITS = CE_OP_MASKED_LOGITS
OP_TOP_M = CE_OP_TOP_M
OP_TOP_M_LOG_SOFTMAX = CE_OP_TOP_M_LOG_SOFTMAX
OP_DRAFT_STEP = CE_OP_DRAFT_STEP
MAX_TOP_M = CE_MAX_TOP_M
