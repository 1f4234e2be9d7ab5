"""Host-side checks of the C ABI (no GPU): symbols, validation, sizing.

ce_head_create, ce_workspace_bytes, ce_head_persistent_bytes and the error
paths of the compute calls make no HIP call, so they run here with fake
(aligned, never dereferenced) device addresses.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from centroid_masked_sparse_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce.h")
FAKE = 0x10000          # aligned fake device address (never dereferenced here)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_ffi.LIB_PATH):
        from centroid_masked_sparse_amd import build_lib
        build_lib.build()
    return _ffi.load()


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _declared_symbols()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", _ffi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(_ffi.SIGNATURES), "binding and header disagree"
    for n in names:
        assert getattr(lib, n) is not None


def _desc(d=64, V=256, Nc=4, max_B=8, max_K=4, dtype=_ffi.CE_BF16, tos=None, off=None,
          c_ptr=FAKE, e_ptr=FAKE, slab=_ffi.CE_SLAB_NATIVE, proj=_ffi.CE_PROJ_AUTO):
    tos = np.arange(V, dtype=np.int32) if tos is None else np.asarray(tos, dtype=np.int32)
    keep = [tos]
    desc = _ffi.HeadDesc(d=d, V=V, Nc=Nc, max_B=max_B, max_K=max_K, dtype=dtype,
                         centroids=c_ptr, emb_ordered=e_ptr,
                         token_of_slot=tos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                         slab_format=slab, projection=proj)
    if off is not None:
        off = np.asarray(off, dtype=np.int32)
        keep.append(off)
        desc.cluster_offsets = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return desc, keep


def _create(lib, desc):
    h = ctypes.c_void_p()
    st = lib.ce_head_create(ctypes.byref(desc), ctypes.byref(h))
    return st, h


ERR = {v: k for k, v in _ffi.STATUS_NAMES.items()}


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), "CE_ERR_BAD_DTYPE"),
    (dict(d=96), "CE_ERR_BAD_SHAPE"),
    (dict(d=0), "CE_ERR_BAD_SHAPE"),
    (dict(Nc=0), "CE_ERR_BAD_SHAPE"),
    (dict(Nc=9000, V=9000 * 2, max_K=4), "CE_ERR_BAD_SHAPE"),
    (dict(max_K=5), "CE_ERR_BAD_SHAPE"),
    (dict(max_B=0), "CE_ERR_BAD_SHAPE"),
    (dict(c_ptr=FAKE + 8), "CE_ERR_MISALIGNED"),
    (dict(e_ptr=FAKE + 2), "CE_ERR_MISALIGNED"),
    (dict(V=250), "CE_ERR_BAD_LAYOUT"),                       # V % Nc with equal clusters
    (dict(tos=[0] * 256), "CE_ERR_BAD_LAYOUT"),               # not a permutation
    (dict(tos=np.arange(1, 257)), "CE_ERR_BAD_LAYOUT"),       # out of range
    (dict(off=[0, 10, 5, 200, 256]), "CE_ERR_BAD_LAYOUT"),    # decreasing
    (dict(off=[0, 10, 20, 30, 255]), "CE_ERR_BAD_LAYOUT"),    # does not end at V
    (dict(off=[1, 10, 20, 30, 256]), "CE_ERR_BAD_LAYOUT"),    # does not start at 0
    (dict(c_ptr=0), "CE_ERR_NULL_POINTER"),
    (dict(slab=2), "CE_ERR_BAD_DTYPE"),
    (dict(slab=_ffi.CE_SLAB_FP8_E4M3, dtype=_ffi.CE_F32), "CE_ERR_BAD_DTYPE"),   # FP8 from bf16 only
    (dict(proj=3), "CE_ERR_BAD_DTYPE"),
    (dict(proj=_ffi.CE_PROJ_MFMA, dtype=_ffi.CE_F32), "CE_ERR_BAD_DTYPE"),      # MFMA for bf16 only
])
def test_create_rejects(lib, kw, want):
    desc, _keep = _desc(**kw)
    st, h = _create(lib, desc)
    assert _ffi.STATUS_NAMES[st] == want
    assert not h.value
    assert lib.ce_last_error().decode()


def test_create_null_args(lib):
    h = ctypes.c_void_p()
    assert lib.ce_head_create(None, ctypes.byref(h)) == ERR["CE_ERR_NULL_POINTER"]
    desc, _keep = _desc()
    assert lib.ce_head_create(ctypes.byref(desc), None) == ERR["CE_ERR_NULL_POINTER"]


def test_create_ragged_and_sizes(lib):
    off = [0, 0, 100, 130, 256]              # an empty cluster and a 100-token one
    tos = np.random.default_rng(0).permutation(256)
    desc, _keep = _desc(tos=tos, off=off, max_B=100, max_K=4)
    st, h = _create(lib, desc)
    assert st == 0
    try:
        n = ctypes.c_size_t()
        assert lib.ce_head_persistent_bytes(h, ctypes.byref(n)) == 0
        # statistics (4 words) + offsets (5 ints) + token_of_slot (V ints) +
        # an empty tile list (clusters of 0, 100, 30 and 126 tokens hold 0, 2,
        # 1 and 2 tiles, so the tiling is the contiguous one: V / 64 = 4
        # tiles) + the tiles' slot tokens (4 x 64 ints) and clusters (4 x 64
        # shorts), each rounded up to 256 bytes, + packed embeddings (4 tiles),
        # their slots' norms (4 x 64 floats) and centroids (1 tile) of 64 rows
        # x 64 bf16
        assert n.value == 256 + 256 + 1024 + 256 + 4 * 256 + 2 * 256 + 4 * 8192 + 4 * 256 + 8192
        assert lib.ce_workspace_bytes(h, 8, 2, _ffi.CE_OP_TOPK, ctypes.byref(n)) == 0
        assert n.value == 0
        sizes = {}
        for op in (_ffi.CE_OP_SCORE, _ffi.CE_OP_TOP_TOKENS, _ffi.CE_OP_MASKED_LOGITS):
            assert lib.ce_workspace_bytes(h, 8, 2, op, ctypes.byref(n)) == 0
            sizes[op] = n.value
            assert n.value % 256 == 0
        assert sizes[_ffi.CE_OP_SCORE] == 0
        # top tokens on a ragged bf16 head adds the certified argmax's row
        # norms (64 floats, one 256-byte region) and records: one of 16 bytes
        # per (row, tile), 8 rows x 4 tiles
        assert sizes[_ffi.CE_OP_TOP_TOKENS] == sizes[_ffi.CE_OP_MASKED_LOGITS] + 256 + 8 * 4 * 16
        # more than one pass of rows needs no more workspace than one full pass
        assert lib.ce_workspace_bytes(h, 64, 2, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(n)) == 0
        one = n.value
        assert lib.ce_workspace_bytes(h, 100, 2, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(n)) == 0
        assert n.value == one
        assert lib.ce_workspace_bytes(h, 101, 2, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(n)) == ERR["CE_ERR_BAD_SHAPE"]
        assert lib.ce_workspace_bytes(h, 8, 5, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(n)) == ERR["CE_ERR_BAD_SHAPE"]
        assert lib.ce_workspace_bytes(h, 8, 0, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(n)) == ERR["CE_ERR_BAD_SHAPE"]
        assert lib.ce_workspace_bytes(h, 8, 1, 9, ctypes.byref(n)) == ERR["CE_ERR_UNSUPPORTED"]
        # top-m: the masked sizes plus its segment lists (tiles the K largest
        # clusters touch: 2 + 2 for K=2, of one 64-token tile's keys each)
        assert lib.ce_workspace_bytes(h, 8, 2, _ffi.CE_OP_TOP_M, ctypes.byref(n)) == 0
        assert n.value >= sizes[_ffi.CE_OP_MASKED_LOGITS] + 8 * 4 * 64 * 8
        # the log-softmax form of top-m takes the same workspace
        n2 = ctypes.c_size_t()
        assert lib.ce_workspace_bytes(h, 8, 2, _ffi.CE_OP_TOP_M_LOG_SOFTMAX, ctypes.byref(n2)) == 0
        assert n2.value == n.value
    finally:
        lib.ce_head_destroy(h)


def test_compute_calls_before_prepare_fail_on_host(lib):
    desc, _keep = _desc()
    st, h = _create(lib, desc)
    assert st == 0
    try:
        NP = ERR["CE_ERR_NOT_PREPARED"]
        assert lib.ce_top_tokens(h, FAKE, 1, 2, FAKE, None, FAKE, 1 << 20, None) == NP
        assert lib.ce_masked_logits(h, FAKE, 1, 2, FAKE, None, FAKE, 1 << 20, None) == NP
        assert lib.ce_top_m(h, FAKE, 1, 2, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == NP
        assert lib.ce_top_m_log_softmax(h, FAKE, 1, 2, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == NP
        assert lib.ce_score_centroids(h, FAKE, 1, FAKE, None) == NP
        assert lib.ce_topk(h, FAKE, 1, 2, FAKE, None) == NP
        assert "prepare" in lib.ce_last_error().decode()
        assert lib.ce_top_tokens(None, FAKE, 1, 2, FAKE, None, FAKE, 1, None) == ERR["CE_ERR_NULL_POINTER"]
        g = ctypes.c_void_p()
        # every check runs before the capture starts: these make no HIP call
        assert lib.ce_graph_capture(h, _ffi.CE_OP_SCORE, FAKE, 1, 2, FAKE, None, FAKE, 1, FAKE,
                                    ctypes.byref(g)) == NP
        assert lib.ce_graph_capture(h, _ffi.CE_OP_TOP_M, FAKE, 1, 2, FAKE, None, FAKE, 1, FAKE,
                                    ctypes.byref(g)) == ERR["CE_ERR_UNSUPPORTED"]
        assert lib.ce_graph_capture(h, 17, FAKE, 1, 2, FAKE, None, FAKE, 1, FAKE,
                                    ctypes.byref(g)) == ERR["CE_ERR_UNSUPPORTED"]
        call = _ffi.CeCall(op=_ffi.CE_OP_TOP_M, in_=FAKE, B=1, K=2, m=4, out=FAKE, out_logits=FAKE,
                           ws=FAKE, ws_bytes=1 << 20)
        assert lib.ce_graph_capture_call(h, None, FAKE, ctypes.byref(g)) == ERR["CE_ERR_NULL_POINTER"]
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), FAKE, None) == ERR["CE_ERR_NULL_POINTER"]
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), None,
                                         ctypes.byref(g)) == ERR["CE_ERR_UNSUPPORTED"]
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), FAKE, ctypes.byref(g)) == NP
        call.op = _ffi.CE_OP_DRAFT_STEP
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), FAKE, ctypes.byref(g)) == NP
        call.op = _ffi.CE_OP_TOP_M_LOG_SOFTMAX
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), FAKE, ctypes.byref(g)) == NP
        call.op = _ffi.CE_OP_TOP_M_LOG_SOFTMAX + 1
        assert lib.ce_graph_capture_call(h, ctypes.byref(call), FAKE,
                                         ctypes.byref(g)) == ERR["CE_ERR_UNSUPPORTED"]
        assert not g.value
        assert lib.ce_graph_launch(None, None) == ERR["CE_ERR_NULL_POINTER"]
        assert lib.ce_graph_destroy(None) == 0
        assert lib.ce_head_prepare(h, None, 0, None) == ERR["CE_ERR_NULL_POINTER"]
        assert lib.ce_head_prepare(h, FAKE + 16, 1 << 20, None) == ERR["CE_ERR_MISALIGNED"]
        assert lib.ce_head_prepare(h, FAKE, 16, None) == ERR["CE_ERR_WORKSPACE_TOO_SMALL"]
        assert lib.ce_probe_gather_events(None, None) == ERR["CE_ERR_NULL_POINTER"]
        counts = (ctypes.c_uint64 * 2)()
        assert lib.ce_head_repair_counts(h, counts) == NP
        assert lib.ce_head_repair_counts(h, None) == ERR["CE_ERR_NULL_POINTER"]
        assert lib.ce_probe_approx_scores(h, FAKE, 1, FAKE, None) == NP
    finally:
        assert lib.ce_head_destroy(h) == 0
    assert lib.ce_head_destroy(None) == 0


def test_status_strings(lib):
    for code, name in _ffi.STATUS_NAMES.items():
        assert lib.ce_status_string(code).decode() == name
    assert lib.ce_status_string(99).decode() == "CE_UNKNOWN_STATUS"


def test_product_path_never_imports_oracle():
    pkg = os.path.join(ROOT, "centroid_masked_sparse_amd")
    for dirpath, _dirs, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "workloads" not in text, f


def test_fp8_slab_sizes(lib):
    """FP8 slabs halve the packed embedding bytes of a bf16 head and add a
    float32 scale per tile row; the workspace does not change."""
    off = [0, 0, 100, 130, 256]
    tos = np.random.default_rng(0).permutation(256)
    sizes = {}
    for slab in (_ffi.CE_SLAB_NATIVE, _ffi.CE_SLAB_FP8_E4M3):
        desc, _keep = _desc(tos=tos, off=off, max_B=100, max_K=4, slab=slab)
        st, h = _create(lib, desc)
        assert st == 0
        try:
            n = ctypes.c_size_t()
            assert lib.ce_head_persistent_bytes(h, ctypes.byref(n)) == 0
            w = ctypes.c_size_t()
            assert lib.ce_workspace_bytes(h, 8, 2, _ffi.CE_OP_TOP_TOKENS, ctypes.byref(w)) == 0
            sizes[slab] = (n.value, w.value)
        finally:
            lib.ce_head_destroy(h)
    native, fp8 = sizes[_ffi.CE_SLAB_NATIVE], sizes[_ffi.CE_SLAB_FP8_E4M3]
    # 4 tiles of 64 rows x 64 elements: 4 * 8192 bytes of bf16 become 4 * 4096
    # bytes of codes plus 4 * 256 bytes of scales (each region 256-aligned)
    assert native[0] - fp8[0] == 4 * 8192 - 4 * 4096 - 4 * 256
    assert native[1] == fp8[1]


def test_stream_read_probe_rejects_bad_arguments(lib):
    """The probe's argument checks come before any HIP call."""
    assert lib.ce_probe_stream_read(None, 1024, FAKE, None) == ERR["CE_ERR_NULL_POINTER"]
    assert lib.ce_probe_stream_read(FAKE, 1024, None, None) == ERR["CE_ERR_NULL_POINTER"]
    assert lib.ce_probe_stream_read(FAKE + 4, 1024, FAKE, None) == ERR["CE_ERR_MISALIGNED"]
    assert lib.ce_probe_stream_read(FAKE, 1000, FAKE, None) == ERR["CE_ERR_MISALIGNED"]
