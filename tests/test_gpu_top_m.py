"""GPU parity of the fused top-m (ce_top_m) against the oracle's top_m.

Token ids must match exactly and logits bit for bit (the canonical key),
including the padding (-1, -inf) of rows with fewer than m candidates.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random, make_workload

pytestmark = pytest.mark.gpu


def _check(head, w, B, K, m):
    torch = torch_mod()
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok, val = head.top_m(to_device(rows(w, B), w.dtype), m, K, topk_out=tk)
    torch.cuda.synchronize()
    tok_o, val_o = oracle.top_m(rows(w, B), w.C, w.E, w.offsets, w.tos, K, m, w.dtype)
    _, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert tk.cpu().numpy().tolist() == sel_o.tolist()
    assert tok.cpu().numpy().tolist() == tok_o.tolist(), (B, K, m)
    assert np.array_equal(val.cpu().numpy().view(np.uint32), val_o.view(np.uint32)), (B, K, m)


@pytest.mark.parametrize("K,m", [(4, 1), (4, 5), (4, 32), (64, 32), (1, 32)])
def test_tiny_config(K, m):
    w = make_workload("tiny")
    _check(make_head(w, max_B=4), w, 3, K, m)


@pytest.mark.parametrize("seed,d,V,Nc,K,B,m,ragged", [
    (41, 128, 8192, 64, 4, 9, 8, False),
    (42, 64, 3000, 40, 3, 7, 16, True),     # ragged clusters, some tiny
    (43, 192, 16384, 256, 16, 64, 32, False),
    (44, 64, 5000, 50, 1, 70, 20, True),    # two passes of rows
    (46, 128, 8192, 64, 4, 3, 8, False),    # clusters of two tiles, by-row launch
    (47, 64, 8192, 64, 4, 70, 12, False),   # equal clusters, two passes of rows
])
def test_random_shapes(seed, d, V, Nc, K, B, m, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=max(64, B), ragged=ragged)
    _check(make_head(w, max_B=B), w, B, K, m)


def test_empty_clusters_pad():
    torch = torch_mod()
    d = 64
    h = np.zeros((2, d), dtype=np.float32)
    h[0, 0] = 1.0
    h[1, 0] = -1.0
    C = np.zeros((4, d), dtype=np.float32)
    C[:, 0] = [5.0, 4.0, -1.0, -2.0]       # row 0 picks clusters 0,1 (empty); row 1 picks 2,3
    E = np.random.default_rng(0).standard_normal((128, d)).astype(np.float32)
    off = np.array([0, 0, 0, 100, 128], dtype=np.int32)   # clusters of 0, 0, 100, 28 tokens
    tos = np.random.default_rng(1).permutation(128).astype(np.int32)
    from centroid_masked_sparse_amd import Head
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, off, max_B=2, max_K=4)
    hd = torch.from_numpy(h).cuda()
    for K, m in ((2, 5), (1, 32), (3, 32)):
        tok, val = head.top_m(hd, m, K)
        tok_o, val_o = oracle.top_m(h, C, E, off, tos, K, m, "f32")
        assert tok.cpu().numpy().tolist() == tok_o.tolist(), (K, m)
        assert np.array_equal(val.cpu().numpy().view(np.uint32), val_o.view(np.uint32)), (K, m)
        if K == 2:
            assert tok_o[0].tolist() == [-1] * m      # row 0 selected only empty clusters


def test_merge_limit_edge():
    """The merge holds a row's segment heads (one per tile of its K clusters)
    and m * 64 candidate keys in 8160 words of LDS.  A head whose largest
    cluster spans 6112 tiles fills it exactly at K = 1, m = 32 (6112 + 2048),
    and is one over it with its second cluster's two tiles at K = 2, m = 32;
    m = 31 fits again.  Row 0 selects the large cluster at K = 1."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import CeError, Head
    d = 64
    big = 6112 * 64
    V = big + 100
    rng = np.random.default_rng(48)
    h = np.zeros((2, d), dtype=np.float32)
    h[:, 1:] = rng.standard_normal((2, d - 1)).astype(np.float32) / 8
    h[0, 0], h[1, 0] = 1.0, -1.0
    C = np.zeros((2, d), dtype=np.float32)
    C[0, 0], C[1, 0] = 1.0, -1.0            # row 0 -> cluster 0 first, row 1 -> cluster 1
    E = (rng.standard_normal((V, d)) / 8).astype(np.float32)
    off = np.array([0, big, V], dtype=np.int32)
    tos = rng.permutation(V).astype(np.int32)
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, off, max_B=2, max_K=2)
    hd = torch.from_numpy(h).cuda()
    for K, m in ((1, 32), (2, 31)):
        tok, val = head.top_m(hd, m, K)
        tok_o, val_o = oracle.top_m(h, C, E, off, tos, K, m, "f32")
        assert tok.cpu().numpy().tolist() == tok_o.tolist(), (K, m)
        assert np.array_equal(val.cpu().numpy().view(np.uint32), val_o.view(np.uint32)), (K, m)
    with pytest.raises(CeError) as e:
        head.top_m(hd, 32, 2)
    assert e.value.status_name == "CE_ERR_UNSUPPORTED"


def test_sweep_config_top8():
    w = make_workload("sweep")
    _check(make_head(w), w, 64, w.K, 8)


def test_bad_m_rejected():
    torch = torch_mod()
    from centroid_masked_sparse_amd import CeError
    w = make_workload("tiny")
    head = make_head(w, max_B=2)
    h = to_device(rows(w, 1), w.dtype)
    for m in (0, 33):
        with pytest.raises(CeError) as e:
            head.top_m(h, m, 4, out=torch.empty((1, max(m, 1)), dtype=torch.int32, device="cuda:0"),
                       logits_out=torch.empty((1, max(m, 1)), dtype=torch.float32, device="cuda:0"))
        assert e.value.status_name == "CE_ERR_BAD_SHAPE"


def test_top_m_under_stream_capture():
    """ce_top_m is capture-safe: a graph captured around it replays to the
    eager result, with eager work and synchronisation between replays."""
    torch = torch_mod()
    w = make_random(45, d=128, V=8192, Nc=64, dtype="bf16", rows=16)
    head = make_head(w, max_B=16)
    h = to_device(rows(w, 16), w.dtype)
    tok_e, val_e = head.top_m(h, 6, 4)
    tok_e, val_e = tok_e.clone(), val_e.clone()
    tok = torch.empty((16, 6), dtype=torch.int32, device="cuda:0")
    val = torch.empty((16, 6), dtype=torch.float32, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        head.top_m(h, 6, 4, out=tok, logits_out=val)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        head.top_m(h, 6, 4, out=tok, logits_out=val)
    for _ in range(3):
        tok.fill_(-5)
        val.fill_(7.0)
        head.top_tokens(h, 4)          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tok, tok_e)
        assert torch.equal(val.view(torch.int32), val_e.view(torch.int32))
