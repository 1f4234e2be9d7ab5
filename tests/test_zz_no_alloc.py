"""ce_top_tokens_static (the entry point that allocates nothing) against
ce_top_tokens, through the C ABI.

Two calls in a row share the library's static per-GPU scratch, the second
with a smaller batch; both must give exactly the tokens and top-K ids of
ce_top_tokens with its own workspace (bit-exact ids, as every parity test).
A call whose workspace exceeds the static scratch is rejected on the host
and writes nothing.
"""

import ctypes

import numpy as np
import pytest

from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu


def _static_call(head, h, K, out, tk):
    torch = torch_mod()
    from centroid_masked_sparse_amd import _ffi
    st = head._lib.ce_top_tokens_static(head._handle, ctypes.c_void_p(h.data_ptr()), h.shape[0], K,
                                        ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(tk.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return _ffi.STATUS_NAMES[st]


def _compare(head, w, B, K):
    torch = torch_mod()
    h = to_device(rows(w, B), w.dtype)
    out = torch.full((B,), -9, dtype=torch.int32, device="cuda:0")
    tk = torch.full((B, K), -9, dtype=torch.int32, device="cuda:0")
    assert _static_call(head, h, K, out, tk) == "CE_SUCCESS"
    tk_ref = torch.full((B, K), -8, dtype=torch.int32, device="cuda:0")
    ref = head.top_tokens(h, K, topk_out=tk_ref)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == ref.cpu().tolist(), B
    assert tk.cpu().tolist() == tk_ref.cpu().tolist(), B


def test_static_scratch_calls_match_top_tokens():
    w = make_workload("sweep")
    head = make_head(w)
    _compare(head, w, 64, w.K)       # the largest batch first
    _compare(head, w, 5, w.K)        # then a smaller one on the same scratch
    # another head, a ragged one, on the same scratch
    r = make_random(95, d=128, V=6000, Nc=70, dtype="bf16", rows=64, ragged=True)
    _compare(make_head(r, max_B=70, max_K=9), r, 70, 9)    # two passes of rows
    _compare(head, w, 1, w.K)


def test_static_scratch_rejects_too_large_a_call():
    """Nc = 8192 with K = Nc needs 4.06 MiB of workspace, more than the
    4 MiB static scratch: rejected before anything is enqueued."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import _ffi
    r = make_random(96, d=64, V=8192, Nc=8192, dtype="bf16", rows=4)
    head = make_head(r, max_B=64, max_K=8192)
    assert head.workspace_bytes(64, 8192, _ffi.CE_OP_TOP_TOKENS) > _ffi.CE_STATIC_SCRATCH_BYTES
    h = to_device(rows(r, 64), r.dtype)
    out = torch.full((64,), -9, dtype=torch.int32, device="cuda:0")
    tk = torch.full((64, 8192), -9, dtype=torch.int32, device="cuda:0")
    assert _static_call(head, h, 8192, out, tk) == "CE_ERR_UNSUPPORTED"
    assert "static scratch" in head._lib.ce_last_error().decode()
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -9).all()
    # a smaller K fits and matches
    _compare(head, r, 64, 300)


def test_static_scratch_takes_the_float64_dot_when_records_do_not_fit():
    """A ragged head of 4096 tiles takes the matrix-core argmax, whose
    records at B = 64 (64 x 4096 x 16 bytes) alone fill the static scratch:
    the static call takes the float64 dot instead, with the same tokens as
    ce_top_tokens (which takes the matrix cores) and the oracle."""
    import oracle
    from centroid_masked_sparse_amd import _ffi
    r = make_random(97, d=64, V=262144, Nc=2048, dtype="bf16", rows=64, ragged=True)
    head = make_head(r, max_B=64, max_K=4)
    assert head.workspace_bytes(64, 4, _ffi.CE_OP_TOP_TOKENS) > _ffi.CE_STATIC_SCRATCH_BYTES
    _compare(head, r, 64, 4)
    _compare(head, r, 7, 4)
    tok_o, _, _ = oracle.top_tokens(rows(r, 7), r.C, r.E, r.offsets, r.tos, 4, r.dtype)
    torch = torch_mod()
    h = to_device(rows(r, 7), r.dtype)
    out = torch.full((7,), -9, dtype=torch.int32, device="cuda:0")
    tk = torch.full((7, 4), -9, dtype=torch.int32, device="cuda:0")
    assert _static_call(head, h, 4, out, tk) == "CE_SUCCESS"
    torch.cuda.synchronize()
    assert out.cpu().tolist() == tok_o.tolist()
