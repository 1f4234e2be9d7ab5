"""GPU parity of ce_top_m_log_softmax: the fused top-m with log-probabilities
under the softmax over each row's candidate set, against the oracle.

Tokens and their order must equal ce_top_m's (and the oracle's) exactly,
padding included.  Log-probabilities are float64 evaluations rounded once to
fp32; the library's summation order of the exponentials differs from the
oracle's, so each value may differ from the oracle's by one fp32 step
(both lie within a fraction of a step of the exact formula), and no more.
Repeated calls and graph replays must agree bit for bit.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu


def _ulps(a, b):
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _compare(tok, lp, tok_o, lp_o, label):
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
    assert tok.tolist() == tok_o.tolist(), label
    pad = tok_o < 0
    assert np.all(np.isneginf(lp[pad])), label
    fin = ~pad
    assert np.all(np.isfinite(lp[fin])), label
    d = _ulps(lp[fin], lp_o[fin])
    assert d.size == 0 or d.max() <= 1, (label, int(d.max()))
    return int((d == 0).sum()), int(d.size)


def _check(head, w, B, K, m, hb=None):
    torch = torch_mod()
    hb = rows(w, B) if hb is None else hb
    h = to_device(hb, w.dtype)
    tok, lp = head.top_m(h, m, K, log_softmax=True)
    tok_m, _ = head.top_m(h, m, K)
    torch.cuda.synchronize()
    tok_o, lp_o = oracle.top_m_log_softmax(hb, w.C, w.E, w.offsets, w.tos, K, m, w.dtype)
    assert tok.cpu().numpy().tolist() == tok_m.cpu().numpy().tolist()
    return _compare(tok, lp, tok_o, lp_o, (B, K, m))


@pytest.mark.parametrize("seed,d,V,Nc,K,B,m,ragged", [
    (141, 128, 8192, 64, 4, 9, 8, False),
    (142, 64, 3000, 40, 3, 7, 16, True),     # ragged clusters, some tiny (counter path)
    (143, 192, 16384, 256, 16, 64, 32, False),
    (144, 64, 5000, 50, 1, 70, 20, True),    # two passes of rows
    (146, 128, 8192, 64, 4, 3, 8, False),    # clusters of two tiles, by-row launch
    (147, 64, 8192, 64, 4, 70, 12, False),   # equal clusters, two passes of rows
])
def test_random_shapes(seed, d, V, Nc, K, B, m, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=max(64, B), ragged=ragged)
    exact, total = _check(make_head(w, max_B=B), w, B, K, m)
    print(f"{exact}/{total} log-probabilities bit-equal to the oracle's")


def test_sweep_config_full_size():
    w = make_workload("sweep")
    exact, total = _check(make_head(w, max_B=64, max_K=w.K), w, 64, w.K, 8)
    print(f"sweep B=64: {exact}/{total} bit-equal")
    assert exact >= 0.9 * total


def test_rows_whose_candidates_all_fit_sum_to_one():
    """m equal to the row's candidate count (two clusters of 16 tokens):
    every candidate is listed, so the probabilities sum to 1."""
    torch = torch_mod()
    w = make_random(150, d=64, V=1024, Nc=64, dtype="bf16", rows=8, ragged=False)
    head = make_head(w, max_B=8)
    K, B = 2, 5
    tok, lp = head.top_m(to_device(rows(w, B), w.dtype), 32, K, log_softmax=True)
    torch.cuda.synchronize()
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy().astype(np.float64)
    for b in range(B):
        assert int((tok[b] >= 0).sum()) == 32
        assert abs(np.exp(lp[b]).sum() - 1.0) < 1e-5
    _check(head, w, B, K, 32)


def test_fp32_head():
    w = make_workload("tiny")
    _check(make_head(w, max_B=4), w, 3, 4, 32)


def test_large_logits_need_the_max_shift():
    """Rows scaled by 64 (exact in bf16) give logits in the hundreds, whose
    exponentials overflow float64 without the shift by the row maximum."""
    from workloads.synth import f32_to_bf16_bits
    w = make_random(148, d=128, V=8192, Nc=64, dtype="bf16", rows=64, ragged=False)
    hb = f32_to_bf16_bits((oracle.upcast(rows(w, 8), "bf16") * 64.0).astype(np.float32))
    _check(make_head(w, max_B=8), w, 8, 4, 16, hb=hb)


def test_fp8_slabs():
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    from oracle import fp8_slabs as f8
    w = make_random(149, d=128, V=8192, Nc=64, dtype="bf16", rows=64, ragged=False)
    B, K, m = 12, 4, 10
    hb = rows(w, B)
    head = Head(to_device(w.C, "bf16"), to_device(w.E, "bf16"), w.tos, max_B=B, max_K=K, slabs="fp8")
    tok, lp = head.top_m(to_device(hb, "bf16"), m, K, log_softmax=True)
    torch.cuda.synchronize()
    codes, sc = f8.quantize_rows(w.E)
    M = f8.masked_logits_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K)
    tok_o, _ = f8.top_m_fp8(hb, w.C, codes, sc, w.offsets, w.tos, K, m)
    lp_o = np.full((B, m), -np.inf, dtype=np.float32)
    for b in range(B):
        fin = np.isfinite(M[b])
        by_token = dict(zip(np.nonzero(fin)[0].tolist(), oracle.log_softmax_candidates(M[b][fin]).tolist()))
        n = int((tok_o[b] >= 0).sum())
        lp_o[b, :n] = [by_token[t] for t in tok_o[b, :n].tolist()]
    _compare(tok, lp, tok_o, lp_o, "fp8")


def test_repeats_and_graph_replays_are_bit_identical():
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_M_LOG_SOFTMAX
    w = make_workload("sweep")
    B, K, m = 16, w.K, 8
    head = make_head(w, max_B=B, max_K=K)
    h = to_device(rows(w, B), w.dtype)
    t1, l1 = head.top_m(h, m, K, log_softmax=True)
    t1, l1 = t1.clone(), l1.clone()
    t2, l2 = head.top_m(h, m, K, log_softmax=True)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    out = torch.empty((B, m), dtype=torch.int32, device="cuda:0")
    lpo = torch.empty((B, m), dtype=torch.float32, device="cuda:0")
    g = head.capture(OP_TOP_M_LOG_SOFTMAX, h, K, out, m=m, logits_out=lpo)
    for i in range(4):
        out.fill_(-7)
        lpo.fill_(0.0)
        head.top_tokens(h, K)            # eager work between replays
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(out, t1), i
        assert torch.equal(lpo.view(torch.int32), l1.view(torch.int32)), i
    g.close()


def test_empty_and_single_candidate_rows():
    """A row whose selected clusters are all empty is padding only; a row
    with one candidate gives it log-probability exactly 0."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    d = 64
    h = np.zeros((3, d), dtype=np.float32)
    h[0, 0] = 1.0    # picks cluster 0 (empty) at K = 1
    h[1, 1] = 1.0    # picks cluster 1 (one token)
    h[2, 2] = 1.0    # picks clusters 2 and 3 at K = 2
    C = np.zeros((4, d), dtype=np.float32)
    C[0, 0] = C[1, 1] = 5.0
    C[2, 2], C[3, 2] = 3.0, 2.0
    E = np.random.default_rng(3).standard_normal((128, d)).astype(np.float32)
    off = np.array([0, 0, 1, 101, 128], dtype=np.int32)   # clusters of 0, 1, 100, 27 tokens
    tos = np.random.default_rng(4).permutation(128).astype(np.int32)
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, off, max_B=3, max_K=4)
    hd = torch.from_numpy(h).cuda()
    for K, m in ((1, 4), (2, 32)):
        tok, lp = head.top_m(hd, m, K, log_softmax=True)
        torch.cuda.synchronize()
        tok_o, lp_o = oracle.top_m_log_softmax(h, C, E, off, tos, K, m, "f32")
        _compare(tok, lp, tok_o, lp_o, (K, m))
        if K == 1:
            assert tok_o[0].tolist() == [-1] * m
            assert tok_o[1, 0] >= 0 and tok_o[1, 1] == -1
            assert lp.cpu().numpy()[1, 0] == 0.0


@pytest.mark.parametrize("ragged", [False, True])
def test_matrix_core_projection(ragged):
    """The MFMA projection with the certified top-K selects the same
    centroids, so tokens and log-probabilities are those of the float64
    projection."""
    w = make_random(151, d=128, V=8192, Nc=64, dtype="bf16", rows=64, ragged=ragged)
    _check(make_head(w, max_B=24, projection="mfma"), w, 24, 4, 8)


def test_closed_form_on_integer_logits():
    """One-hot rows and embeddings whose first element is 0, 1, 2 or 3 give
    exact integer logits: the row's 64 candidates hold each value 16 times,
    so log p(l) = l - log(16 (1 + e + e^2 + e^3)), and the m best are the
    lowest-id tokens of logit 3 (ties by token id)."""
    import math
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    d, V = 64, 128
    C = np.zeros((2, d), dtype=np.float32)
    C[0, 0], C[1, 0] = 1.0, -1.0            # the row selects cluster 0 at K = 1
    E = np.zeros((V, d), dtype=np.float32)
    E[:64, 0] = np.arange(64) % 4           # cluster 0: logits 0, 1, 2, 3, ...
    E[64:, 0] = 5.0
    tos = np.random.default_rng(8).permutation(V).astype(np.int32)
    h = np.zeros((2, d), dtype=np.float32)
    h[:, 0] = 1.0
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, max_B=2, max_K=2)
    m = 8
    tok, lp = head.top_m(torch.from_numpy(h).cuda(), m, 1, log_softmax=True)
    torch.cuda.synchronize()
    lse = math.log(16.0 * (1.0 + math.e + math.e ** 2 + math.e ** 3))
    want_tok = sorted(int(tos[j]) for j in range(64) if j % 4 == 3)[:m]
    for b in range(2):
        assert tok.cpu().numpy()[b].tolist() == want_tok
        got = lp.cpu().numpy()[b]
        assert np.all(_ulps(got, np.full(m, np.float32(3.0 - lse))) <= 1), got


def test_every_token_a_candidate_is_the_dense_log_softmax():
    """K = Nc: every token is a candidate, so the log-probabilities are the
    full-vocabulary log-softmax of the dense logits."""
    torch = torch_mod()
    w = make_workload("tiny")
    B, K, m = 3, w.Nc, 32
    head = make_head(w, max_B=4)
    hb = rows(w, B)
    tok, lp = head.top_m(to_device(hb, w.dtype), m, K, log_softmax=True)
    torch.cuda.synchronize()
    dense = oracle.dense_logits(hb, w.E, w.tos, w.dtype)
    tok_o, lp_o = oracle.top_m_log_softmax(hb, w.C, w.E, w.offsets, w.tos, K, m, w.dtype)
    _compare(tok, lp, tok_o, lp_o, "K=Nc")
    for b in range(B):
        full = oracle.log_softmax_candidates(dense[b])
        assert np.all(_ulps(lp.cpu().numpy()[b], full[tok_o[b]]) <= 1)
