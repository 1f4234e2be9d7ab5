"""Graph replay against the oracle: every captured batch size of the sweep,
the forward rows, every op through ce_graph_capture_call, and determinism
over many replays.

The page's proposer captures one CUDA graph per batch size in {1, 2, 4, 8,
16, 32, 64} and replays the next larger one (Gemma4Proposer
._setup_centroids_cuda_graphs, vLLM compare view, diff of
spec_decode/gemma4.py).  Here each size's graph is compared with the oracle
on every replay, with eager calls and synchronisation in between.
"""

import numpy as np
import pytest

import oracle
from oracle import draft as od
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import CONFIGS, make_random, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sweep():
    w = make_workload("sweep")
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    return w, make_head(w), tok_o, sel_o


@pytest.mark.parametrize("B", CONFIGS["sweep"].batches)
def test_sweep_graph_every_size_against_oracle(sweep, B):
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    w, head, tok_o, sel_o = sweep
    h = to_device(rows(w, B), w.dtype)
    out = torch.full((B,), -9, dtype=torch.int32, device="cuda:0")
    tk = torch.full((B, w.K), -9, dtype=torch.int32, device="cuda:0")
    g = head.capture(OP_TOP_TOKENS, h, w.K, out, topk_out=tk)
    for i in range(3):
        out.fill_(-9)
        tk.fill_(-9)
        g.launch()
        torch.cuda.synchronize()
        assert out.cpu().tolist() == tok_o[:B].tolist(), (B, i)
        assert tk.cpu().tolist() == sel_o[:B].tolist(), (B, i)
        head.top_tokens(h[: max(1, B // 2)], w.K)     # eager work between replays
        torch.cuda.synchronize()
    g.close()


def test_forward_graphs_against_oracle(sweep):
    """The masked configuration's sizes (B = 1, 16, 64), replayed: every
    entry of every row, the -inf pattern included, equals the oracle's."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_MASKED_LOGITS
    w, head, _, sel_o = sweep
    M_o, _ = oracle.masked_logits(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    want = M_o.view(np.uint32)
    for B in CONFIGS["masked"].batches:
        h = to_device(rows(w, B), w.dtype)
        out = torch.empty((B, w.V), dtype=torch.float32, device="cuda:0")
        tk = torch.empty((B, w.K), dtype=torch.int32, device="cuda:0")
        g = head.capture(OP_MASKED_LOGITS, h, w.K, out, topk_out=tk)
        for i in range(2):
            out.fill_(7.0)
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want[:B]), (B, i)
            assert tk.cpu().tolist() == sel_o[:B].tolist(), (B, i)
        g.close()
        del out


@pytest.mark.parametrize("B", [1, 64])
def test_hundred_replays_bit_identical(sweep, B):
    """100 replays of one graph give the same tokens and ids every time (no
    state leaks from one replay into the next), and those are the oracle's."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    w, head, tok_o, sel_o = sweep
    h = to_device(rows(w, B), w.dtype)
    out = torch.empty((B,), dtype=torch.int32, device="cuda:0")
    tk = torch.empty((B, w.K), dtype=torch.int32, device="cuda:0")
    g = head.capture(OP_TOP_TOKENS, h, w.K, out, topk_out=tk)
    outs = torch.empty((100, B), dtype=torch.int32, device="cuda:0")
    tks = torch.empty((100, B, w.K), dtype=torch.int32, device="cuda:0")
    for i in range(100):
        g.launch()
        outs[i].copy_(out)
        tks[i].copy_(tk)
    torch.cuda.synchronize()
    o, t = outs.cpu().numpy(), tks.cpu().numpy()
    assert (o == tok_o[:B][None, :]).all()
    assert (t == sel_o[:B][None, :, :]).all()
    g.close()


def test_every_op_through_capture_call():
    """ce_graph_capture_call on a random head: the projection, the top-K on
    given scores, the fused top-m and the fused draft step replay to the
    oracle's values, bit for bit, with eager calls between replays."""
    torch = torch_mod()
    import centroid_masked_sparse_amd as cms
    w = make_random(71, d=128, V=8192, Nc=64, dtype="bf16", rows=64)
    head = make_head(w, max_B=16)
    B, K, m = 12, 5, 9
    hB = rows(w, B)
    h = to_device(hB, w.dtype)

    S = torch.empty((B, w.Nc), dtype=torch.float32, device="cuda:0")
    g_s = head.capture(cms.OP_SCORE, h, None, S)
    S_o = oracle.centroid_scores(hB, w.C, w.dtype)
    ids = torch.empty((B, K), dtype=torch.int32, device="cuda:0")
    S_in = torch.from_numpy(S_o).to("cuda:0")
    g_k = head.capture(cms.OP_TOPK, S_in, K, ids)
    tok = torch.empty((B, m), dtype=torch.int32, device="cuda:0")
    val = torch.empty((B, m), dtype=torch.float32, device="cuda:0")
    g_m = head.capture(cms.OP_TOP_M, h, K, tok, m=m, logits_out=val)
    tok_o, val_o = oracle.top_m(hB, w.C, w.E, w.offsets, w.tos, K, m, w.dtype)

    rng = np.random.default_rng(72)
    from workloads.synth import f32_to_bf16_bits
    x = f32_to_bf16_bits((2.0 * rng.standard_normal((B, w.d))).astype(np.float32))
    nw = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32))
    table = f32_to_bf16_bits(rng.standard_normal((w.V, 32)).astype(np.float32))
    xd, nwd, td = to_device(x, "bf16"), to_device(nw, "bf16"), to_device(table, "bf16")
    h_out = torch.empty_like(xd)
    dtok = torch.empty(B, dtype=torch.int32, device="cuda:0")
    emb = torch.empty((B, 32), dtype=xd.dtype, device="cuda:0")
    g_d = head.capture(cms.OP_DRAFT_STEP, xd, K, dtok, norm_weight=nwd, eps=1e-6, h_out=h_out,
                       emb_table=td, normalizer=3.0, emb_out=emb)
    hn_o, dtok_o, emb_o, _ = od.draft_step(x, nw, 1e-6, w.C, w.E, w.offsets, w.tos, K, table, 3.0,
                                           "bf16")
    sel_o = oracle.topk_centroids(S_o, K)
    for i in range(3):
        for t in (S, val):
            t.fill_(5.0)
        for t in (ids, tok, dtok):
            t.fill_(-3)
        h_out.zero_()
        emb.zero_()
        for g in (g_s, g_k, g_m, g_d):
            g.launch()
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy().view(np.uint32), S_o.view(np.uint32)), i
        assert ids.cpu().tolist() == sel_o.tolist(), i
        assert tok.cpu().tolist() == tok_o.tolist(), i
        assert np.array_equal(val.cpu().numpy().view(np.uint32), val_o.view(np.uint32)), i
        assert np.array_equal(h_out.view(torch.int16).cpu().numpy().view(np.uint16), hn_o), i
        assert dtok.cpu().tolist() == dtok_o.tolist(), i
        assert np.array_equal(emb.view(torch.int16).cpu().numpy().view(np.uint16), emb_o), i
        head.top_m(h[:3], 4, K)              # eager work between replays
        torch.cuda.synchronize()
    for g in (g_s, g_k, g_m, g_d):
        g.close()


def test_capture_errors_leave_no_capture():
    """A call that fails its checks under capture returns its own status and
    leaves the stream able to capture again."""
    torch = torch_mod()
    import centroid_masked_sparse_amd as cms
    from centroid_masked_sparse_amd import CeError
    w = make_random(73, d=64, V=4096, Nc=32, dtype="bf16", rows=8)
    head = make_head(w, max_B=8, max_K=4)
    h = to_device(rows(w, 4), w.dtype)
    tok = torch.empty((4, 8), dtype=torch.int32, device="cuda:0")
    val = torch.empty((4, 8), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    with pytest.raises(CeError) as e:
        head.capture(cms.OP_TOP_M, h, 4, tok, m=40, logits_out=val, stream=s)   # m > 32
    assert e.value.status_name == "CE_ERR_BAD_SHAPE"
    with pytest.raises(CeError) as e:
        head.capture(cms.OP_TOP_TOKENS, h, 9, tok[:, 0].contiguous(), stream=s)   # K > max_K
    assert e.value.status_name == "CE_ERR_BAD_SHAPE"
    g = head.capture(cms.OP_TOP_M, h, 4, tok, m=8, logits_out=val, stream=s)
    g.launch()
    torch.cuda.synchronize()
    tok_o, _ = oracle.top_m(rows(w, 4), w.C, w.E, w.offsets, w.tos, 4, 8, w.dtype)
    assert tok.cpu().tolist() == tok_o.tolist()
    g.close()
