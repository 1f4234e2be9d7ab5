"""ctypes declarations of the C ABI in ``include/ce.h`` (``libce.so``)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libce.so")

CE_SUCCESS = 0
STATUS_NAMES = {
    0: "CE_SUCCESS", 1: "CE_ERR_NULL_POINTER", 2: "CE_ERR_BAD_SHAPE", 3: "CE_ERR_BAD_DTYPE",
    4: "CE_ERR_MISALIGNED", 5: "CE_ERR_BAD_LAYOUT", 6: "CE_ERR_WORKSPACE_TOO_SMALL",
    7: "CE_ERR_NOT_PREPARED", 8: "CE_ERR_HIP", 9: "CE_ERR_UNSUPPORTED",
}
CE_F32, CE_BF16 = 0, 1
CE_OP_SCORE, CE_OP_TOPK, CE_OP_TOP_TOKENS, CE_OP_MASKED_LOGITS, CE_OP_TOP_M = 0, 1, 2, 3, 4
CE_OP_DRAFT_STEP = 5
CE_OP_TOP_M_LOG_SOFTMAX = 6
CE_MAX_TOP_M = 32
CE_STATIC_SCRATCH_BYTES = 4 << 20
CE_SLAB_NATIVE, CE_SLAB_FP8_E4M3 = 0, 1
CE_PROJ_AUTO, CE_PROJ_EXACT, CE_PROJ_MFMA = 0, 1, 2

# Every symbol the header declares, with (restype, argtypes).
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class HeadDesc(ctypes.Structure):
    _fields_ = [
        ("d", _i32), ("V", _i32), ("Nc", _i32), ("max_B", _i32), ("max_K", _i32),
        ("dtype", _i32), ("centroids", _vp), ("emb_ordered", _vp),
        ("cluster_offsets", ctypes.POINTER(_i32)), ("token_of_slot", ctypes.POINTER(_i32)),
        ("slab_format", _i32), ("projection", _i32),
    ]


class CeCall(ctypes.Structure):
    """``ce_call``: one call of any op, for ``ce_graph_capture_call``."""
    _fields_ = [
        ("op", _i32), ("in_", _vp), ("B", _i32), ("K", _i32), ("m", _i32), ("out", _vp),
        ("out_logits", _vp), ("topk_ids", _vp), ("ws", _vp), ("ws_bytes", _sz),
        ("norm_weight", _vp), ("eps", ctypes.c_float), ("h_out", _vp), ("emb_table", _vp),
        ("emb_dim", _i32), ("normalizer", ctypes.c_float), ("emb_out", _vp),
    ]


SIGNATURES = {
    "ce_head_create": (_i32, [ctypes.POINTER(HeadDesc), ctypes.POINTER(_vp)]),
    "ce_head_destroy": (_i32, [_vp]),
    "ce_head_persistent_bytes": (_i32, [_vp, ctypes.POINTER(_sz)]),
    "ce_head_prepare": (_i32, [_vp, _vp, _sz, _vp]),
    "ce_workspace_bytes": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "ce_score_centroids": (_i32, [_vp, _vp, _i32, _vp, _vp]),
    "ce_topk": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "ce_top_tokens": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "ce_top_tokens_static": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "ce_masked_logits": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "ce_top_m": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ce_top_m_log_softmax": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ce_draft_step": (_i32, [_vp, _vp, _vp, ctypes.c_float, _i32, _i32, _vp, _vp, _vp, _i32,
                             ctypes.c_float, _vp, _vp, _vp, _sz, _vp]),
    "ce_graph_capture": (_i32, [_vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp,
                                ctypes.POINTER(_vp)]),
    "ce_graph_capture_call": (_i32, [_vp, ctypes.POINTER(CeCall), _vp, ctypes.POINTER(_vp)]),
    "ce_graph_launch": (_i32, [_vp, _vp]),
    "ce_graph_destroy": (_i32, [_vp]),
    "ce_probe_gather_events": (_i32, [_vp, _vp]),
    "ce_probe_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "ce_head_repair_counts": (_i32, [_vp, ctypes.POINTER(ctypes.c_uint64)]),
    "ce_probe_approx_scores": (_i32, [_vp, _vp, _i32, _vp, _vp]),
    "ce_status_string": (ctypes.c_char_p, [_i32]),
    "ce_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load ``libce.so``.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its bundled HIP runtime then satisfies libce's
    # libamdhip64.so.7 dependency, so one runtime serves both.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
            "python -m centroid_masked_sparse_amd.build_lib")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class CeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{where}: {self.status_name}: {detail}")


def check(status: int, where: str) -> None:
    if status != CE_SUCCESS:
        detail = load().ce_last_error().decode(errors="replace")
        raise CeError(status, where, detail)
