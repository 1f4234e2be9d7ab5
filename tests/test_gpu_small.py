"""GPU parity on small and edge-case inputs, through the C ABI.

Expected values come only from the CPU oracle on the same seeded inputs.
Bar: top-K ids and token ids bit-exact; logits and scores bit-exact as well
(the kernels compute the oracle's canonical rounding), which is checked
together with the 2e-3 abs/rel tolerance that bounds any fp32 result.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import f32_bits, make_head, rows, to_device, torch_mod
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _assert_close_and_exact(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(np.abs(got[fin] - want[fin]) <= TOL + TOL * np.abs(want[fin]))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _topk_ids(head, w, hB, K):
    torch = torch_mod()
    B = hB.shape[0]
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(to_device(hB, w.dtype), K, topk_out=tk)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), tk.cpu().numpy()


def test_tiny_config_scores_topk_tokens_masked():
    w = make_workload("tiny")
    head = make_head(w)
    hB = rows(w, 1)
    for K in (4, 64):
        tok_o, sel_o, _ = oracle.top_tokens(hB, w.C, w.E, w.offsets, w.tos, K, w.dtype)
        tok, tk = _topk_ids(head, w, hB, K)
        assert tk.tolist() == sel_o.tolist()
        assert tok.tolist() == tok_o.tolist()
        M_o, _ = oracle.masked_logits(hB, w.C, w.E, w.offsets, w.tos, K, w.dtype)
        M = head.masked_logits(to_device(hB, w.dtype), K)
        _assert_close_and_exact(M.cpu().numpy(), M_o)
    S = head.score_centroids(to_device(rows(w, 64), w.dtype)).cpu().numpy()
    _assert_close_and_exact(S, oracle.centroid_scores(rows(w, 64), w.C, w.dtype))


@pytest.mark.parametrize("Nc,K,B", [(64, 1, 1), (64, 64, 3), (100, 7, 5), (2048, 32, 64),
                                    (4096, 64, 65), (8192, 300, 2), (2048, 2048, 2)])
def test_topk_bit_exact_with_ties(Nc, K, B):
    torch = torch_mod()
    rng = np.random.default_rng(Nc + K + B)
    w = make_random(1, d=64, V=Nc * 2, Nc=Nc, dtype="bf16", rows=1)
    head = make_head(w, max_B=max(B, 64), max_K=K)
    S = (rng.integers(-6, 7, size=(B, Nc)) * 0.25).astype(np.float32)
    S[S == 0] = np.where(rng.random(int((S == 0).sum())) < 0.5, -0.0, 0.0)
    S[:, ::7] = rng.standard_normal((B, S[:, ::7].shape[1])).astype(np.float32)
    S[0, : min(Nc, 40)] = np.float32(np.inf if B > 4 else -np.inf)
    got = head.topk(torch.from_numpy(S).to("cuda:0"), K).cpu().numpy()
    want = oracle.topk_centroids(S, K)
    assert got.tolist() == want.tolist()


@pytest.mark.parametrize("dtype,d,V,Nc,K,B,ragged", [
    ("bf16", 256, 8192, 64, 4, 37, False),
    ("bf16", 64, 3000, 47, 5, 20, True),
    ("f32", 128, 4096, 32, 3, 9, False),
    ("bf16", 512, 20000, 100, 10, 64, True),
    ("bf16", 64, 4096, 64, 8, 100, False),     # two passes of rows
])
def test_random_shapes_tokens_and_masked(dtype, d, V, Nc, K, B, ragged):
    w = make_random(21 + d + Nc, d=d, V=V, Nc=Nc, dtype=dtype, rows=64, ragged=ragged)
    head = make_head(w, max_B=128)
    hB = rows(w, B)
    tok_o, sel_o, _ = oracle.top_tokens(hB, w.C, w.E, w.offsets, w.tos, K, dtype)
    tok, tk = _topk_ids(head, w, hB, K)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()
    M_o, _ = oracle.masked_logits(hB, w.C, w.E, w.offsets, w.tos, K, dtype)
    M = head.masked_logits(to_device(hB, dtype), K)
    _assert_close_and_exact(M.cpu().numpy(), M_o)


def test_canonical_order_adversarial_rows():
    """Rows whose float64 sum depends on the summation order and rounding."""
    torch = torch_mod()
    d, Nc = 64, 4
    C = np.zeros((Nc, d), dtype=np.float32)
    C[:, :3] = 1.0
    E = np.zeros((Nc * 64, d), dtype=np.float32)
    E[:, :3] = 1.0
    h = np.zeros((4, d), dtype=np.float32)
    h[0, :3] = [2.0 ** 60, 1.0, -2.0 ** 60]          # sequential: +0, exact: 1
    h[1, :3] = [1.0, 2.0 ** 60, -2.0 ** 60]          # sequential: +0
    h[2, :3] = [2.0 ** 60, -2.0 ** 60, 1.0]          # sequential: 1
    h[3, :2] = [1.0, 2.0 ** -24]                     # tie to even: 1
    C[1, 0] = 0.5                                    # make centroid scores differ
    tos = np.random.default_rng(3).permutation(Nc * 64).astype(np.int32)
    from centroid_masked_sparse_amd import Head
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, max_B=4, max_K=Nc)
    S = head.score_centroids(torch.from_numpy(h).cuda()).cpu().numpy()
    want = oracle.centroid_scores(h, C, "f32")
    assert np.array_equal(S.view(np.uint32), want.view(np.uint32))
    assert S[0, 0] == 0.0 and S[2, 0] == 1.0 and S[3, 0] == 1.0
    M = head.masked_logits(torch.from_numpy(h).cuda(), 2).cpu().numpy()
    M_o, _ = oracle.masked_logits(h, C, E, np.arange(Nc + 1) * 64, tos, 2, "f32")
    assert np.array_equal(M.view(np.uint32), M_o.view(np.uint32))


def test_empty_clusters_give_minus_one():
    torch = torch_mod()
    d = 64
    h = np.zeros((2, d), dtype=np.float32)
    h[0, 0] = 1.0
    h[1, 0] = -1.0
    C = np.zeros((4, d), dtype=np.float32)
    C[:, 0] = [5.0, 4.0, -1.0, -2.0]       # row 0 picks clusters 0,1 (empty); row 1 picks 2,3
    E = np.random.default_rng(0).standard_normal((128, d)).astype(np.float32)
    off = np.array([0, 0, 0, 64, 128], dtype=np.int32)
    tos = np.random.default_rng(1).permutation(128).astype(np.int32)
    from centroid_masked_sparse_amd import Head
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, off, max_B=2, max_K=4)
    hd = torch.from_numpy(h).cuda()
    tok = head.top_tokens(hd, 2).cpu().numpy()
    tok_o, _, _ = oracle.top_tokens(h, C, E, off, tos, 2, "f32")
    assert tok_o[0] == -1 and tok.tolist() == tok_o.tolist()
    tok1 = head.top_tokens(hd[:1], 2).cpu().numpy()       # no work item at all
    assert tok1.tolist() == [-1]
    M = head.masked_logits(hd, 2).cpu().numpy()
    M_o, _ = oracle.masked_logits(h, C, E, off, tos, 2, "f32")
    assert np.array_equal(M.view(np.uint32), M_o.view(np.uint32))


def test_zero_batch_writes_nothing():
    torch = torch_mod()
    w = make_workload("tiny")
    head = make_head(w)
    out = torch.full((4,), 12345, dtype=torch.int32, device="cuda:0")
    h0 = to_device(rows(w, 1), w.dtype)[:0]
    head.top_tokens(h0, 4, out=out[:0])
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [12345] * 4


def test_errors_from_device_calls():
    from centroid_masked_sparse_amd import CeError, _ffi
    torch = torch_mod()
    w = make_workload("tiny")
    head = make_head(w, max_B=4, max_K=8)
    h = to_device(rows(w, 5), w.dtype)
    with pytest.raises(CeError) as e:
        head.top_tokens(h, 4)
    assert e.value.status_name == "CE_ERR_BAD_SHAPE"
    with pytest.raises(CeError) as e:
        head.top_tokens(h[:2], 9)
    assert e.value.status_name == "CE_ERR_BAD_SHAPE"
    small = torch.empty(256, dtype=torch.uint8, device="cuda:0")
    out = torch.empty(2, dtype=torch.int32, device="cuda:0")
    st = head._lib.ce_top_tokens(head._handle, h.data_ptr(), 2, 4, out.data_ptr(), None,
                                 small.data_ptr(), small.numel(), None)
    assert _ffi.STATUS_NAMES[st] == "CE_ERR_WORKSPACE_TOO_SMALL"


def test_graph_replay_matches_eager():
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_MASKED_LOGITS, OP_TOP_TOKENS
    w = make_random(31, d=256, V=16384, Nc=128, dtype="bf16", rows=64)
    head = make_head(w)
    h = to_device(rows(w, 8), w.dtype)
    eager_tok = head.top_tokens(h, 8).clone()
    eager_M = head.masked_logits(h[:4], 8).clone()
    out_tok = torch.empty(8, dtype=torch.int32, device="cuda:0")
    out_M = torch.empty((4, w.V), dtype=torch.float32, device="cuda:0")
    hM = h[:4].clone()
    g1 = head.capture(OP_TOP_TOKENS, h, 8, out_tok)
    g2 = head.capture(OP_MASKED_LOGITS, hM, 8, out_M)
    for i in range(4):
        out_tok.fill_(-5)
        out_M.zero_()
        g1.launch()
        g2.launch()
        torch.cuda.synchronize()
        assert torch.equal(out_tok, eager_tok), i
        assert torch.equal(out_M.view(torch.int32), eager_M.view(torch.int32)), i
        _ = head.top_tokens(h, 3)            # eager work between replays
        torch.cuda.synchronize()
    # new inputs at the captured address are picked up by the next replay
    h2 = to_device(rows(w, 16)[8:16], w.dtype)
    h.copy_(h2)
    g1.launch()
    torch.cuda.synchronize()
    assert torch.equal(out_tok, head.top_tokens(h2, 8))
    g1.close()
    g2.close()


def test_stream_read_probe_runs():
    """The streaming-read probe completes on buffers from one vector to a few
    MiB with ragged remainders; all-zero data never matches its store pattern."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import _ffi
    lib = _ffi.load()
    stream = torch.cuda.current_stream().cuda_stream
    for n in (16, 4096 + 16, 1 << 20, (3 << 20) + 48):
        buf = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
        sink = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
        _ffi.check(lib.ce_probe_stream_read(buf.data_ptr(), n, sink.data_ptr(), stream), "probe")
        torch.cuda.synchronize()
        assert sink.item() == 7


def test_probe_events_bracket_gather():
    torch = torch_mod()
    from centroid_masked_sparse_amd import _ffi
    w = make_workload("tiny")
    head = make_head(w)
    h = to_device(rows(w, 1), w.dtype)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    e.record()
    torch.cuda.synchronize()
    _ffi.check(head._lib.ce_probe_gather_events(s.cuda_event, e.cuda_event), "probe")
    head.top_tokens(h, 4)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    assert 0.0 < ms < 100.0
