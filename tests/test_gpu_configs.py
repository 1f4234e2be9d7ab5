"""GPU parity at the full sizes of the five benchmark configurations.

The oracle runs on the same seeded arrays.  Where a full oracle pass would
take too long (the K = Nc check of the wide config) it computes sampled rows.
The sweep also runs through captured HIP graphs, the launch configuration the
benchmark times.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _run_tokens(head, w, B, K):
    torch = torch_mod()
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(to_device(rows(w, B), w.dtype), K, topk_out=tk)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), tk.cpu().numpy()


@pytest.fixture(scope="module")
def sweep():
    w = make_workload(2)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    return w, make_head(w), tok_o, sel_o


def test_sweep_every_batch_size(sweep):
    w, head, tok_o, sel_o = sweep
    for B in CONFIGS[2].batches:
        tok, tk = _run_tokens(head, w, B, w.K)
        assert tk.tolist() == sel_o[:B].tolist(), B
        assert tok.tolist() == tok_o[:B].tolist(), B


def test_sweep_graph_replay(sweep):
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    w, head, tok_o, _ = sweep
    for B in (1, 64):
        h = to_device(rows(w, B), w.dtype)
        out = torch.full((B,), -9, dtype=torch.int32, device="cuda:0")
        g = head.capture(OP_TOP_TOKENS, h, w.K, out)
        for _ in range(3):
            out.fill_(-9)
            g.launch()
            torch.cuda.synchronize()
            assert out.cpu().tolist() == tok_o[:B].tolist()
        g.close()


def test_masked_config_full_rows(sweep):
    w, head, _, sel_o = sweep
    M_o, _ = oracle.masked_logits(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    for B in CONFIGS[3].batches:
        M = head.masked_logits(to_device(rows(w, B), w.dtype), w.K).cpu().numpy()
        assert np.array_equal(M.view(np.uint32), M_o[:B].view(np.uint32)), B
        assert np.all(np.isfinite(M).sum(axis=1) == w.K * (w.V // w.Nc))


def test_wide_config_K64_and_full_K():
    w = make_workload(4)
    head = make_head(w)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    tok, tk = _run_tokens(head, w, 64, w.K)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()
    # K = Nc: every centroid is selected, so the sparse argmax is the dense one
    tok_full, _ = _run_tokens(head, w, 64, w.Nc)
    sample = [0, 17, 42, 63]
    D = oracle.dense_logits(rows(w, 64)[sample], w.E, w.tos, w.dtype)
    assert tok_full[sample].tolist() == np.argmax(D, axis=1).tolist()


def test_skewed_config():
    w = make_workload(5)
    head = make_head(w)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    tok, tk = _run_tokens(head, w, 64, w.K)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()
    # rows of one anchor group share most of their selected centroids
    g = w.groups
    same = [len(set(sel_o[a]) & set(sel_o[b])) / w.K
            for a in range(64) for b in range(a + 1, 64) if g[a] == g[b]]
    assert np.mean(same) > 0.2
