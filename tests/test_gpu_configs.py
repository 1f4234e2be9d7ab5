"""GPU parity at the full sizes of the five benchmark configurations.

The oracle runs on the same seeded arrays.  The dense argmax of the wide
configuration (its K = Nc check), a few minutes of oracle time, is stored for
all 64 rows by tests/golden/make_wide_dense.py.  Graph replays of every
captured size are in test_gpu_graphs.py.
"""

import json
import os

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
    w = make_workload("sweep")
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    return w, make_head(w), tok_o, sel_o


def test_sweep_every_batch_size(sweep):
    w, head, tok_o, sel_o = sweep
    for B in CONFIGS["sweep"].batches:
        tok, tk = _run_tokens(head, w, B, w.K)
        assert tk.tolist() == sel_o[:B].tolist(), B
        assert tok.tolist() == tok_o[:B].tolist(), B


def test_masked_config_full_rows(sweep):
    w, head, _, sel_o = sweep
    M_o, _ = oracle.masked_logits(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    for B in CONFIGS["masked"].batches:
        M = head.masked_logits(to_device(rows(w, B), w.dtype), w.K).cpu().numpy()
        assert np.array_equal(M.view(np.uint32), M_o[:B].view(np.uint32)), B
        assert np.all(np.isfinite(M).sum(axis=1) == w.K * (w.V // w.Nc))


WIDE_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wide_dense.json")


@pytest.fixture(scope="module")
def wide():
    """The wide workload and the oracle's dense argmax of its 64 rows, stored
    by tests/golden/make_wide_dense.py (a few minutes of oracle time)."""
    w = make_workload("wide")
    with open(WIDE_GOLDEN) as f:
        gold = json.load(f)["rows"]
    assert [r["row"] for r in gold] == list(range(64))
    return w, gold


def test_wide_config_K64_and_full_K(wide):
    w, gold = wide
    head = make_head(w)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    tok, tk = _run_tokens(head, w, 64, w.K)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()
    # K = Nc: every centroid is selected, so on every row the sparse argmax
    # is the dense one
    tok_full, tk_full = _run_tokens(head, w, 64, w.Nc)
    assert (tk_full == np.arange(w.Nc)[None, :]).all()
    assert tok_full.tolist() == [r["best"] for r in gold]


def test_wide_dense_comparison_path(wide):
    """The dense comparison path the benchmark times (vendor bf16 GEMM with
    fp32 output over all V tokens, then argmax) against the oracle's dense
    argmax.  Its fp32 sums follow the library's order, so a row is checked
    only where the oracle's two best logits differ by more than twice the
    worst-case fp32 summation error, d*2^-24/(1-d*2^-24) * sum|h_k e_k| plus
    an ulp, of either token."""
    torch = torch_mod()
    w, gold = wide
    inv = np.argsort(w.tos)
    E_tok = to_device(np.ascontiguousarray(w.E[inv]), w.dtype)
    h = to_device(rows(w, 64), w.dtype)
    tok = torch.argmax(torch.mm(E_tok, h.t().contiguous(), out_dtype=torch.float32), dim=0)
    tok = tok.cpu().numpy()
    del E_tok
    H64 = oracle.upcast(rows(w, 64), w.dtype)
    u = 2.0 ** -24
    gamma = w.d * u / (1 - w.d * u)
    checked = 0
    for b, r in enumerate(gold):
        t1, t2 = r["best"], r["second"]
        l1 = float(np.uint32(int(r["best_logit"], 16)).view(np.float32))
        l2 = float(np.uint32(int(r["second_logit"], 16)).view(np.float32))
        bound = 0.0
        for t, lv in ((t1, l1), (t2, l2)):
            e = oracle.upcast(w.E[inv[t]][None, :], w.dtype)[0]
            bound = max(bound, gamma * float(np.abs(H64[b] * e).sum()) + u * abs(lv))
        if l1 - l2 > 2 * bound:
            assert int(tok[b]) == t1, (b, int(tok[b]), t1)
            checked += 1
    # the margins of this draw certify every row (a CPU fact of the stored
    # values and the inputs, not of the GPU)
    assert checked == 64


def test_skewed_config():
    w = make_workload("skewed")
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
