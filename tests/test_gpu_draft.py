"""GPU parity of the fused draft step (ce_draft_step) against the oracle.

The normalised rows, the selected centroids, the tokens and the scaled
embeddings must all match the oracle bit for bit.
"""

import numpy as np
import pytest

from oracle import draft as od
from tests.gpu_helpers import make_head, to_device, torch_mod
from workloads import make_random, make_workload
from workloads.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(seed, B, d, V, emb_dim, dtype):
    """Pre-norm rows x ~ N(0, 4), norm weight 1 + N(0, 0.01), an embedding
    table ~ N(0, 1) of emb_dim columns indexed by token id."""
    rng = np.random.default_rng(seed)
    cast = (lambda a: f32_to_bf16_bits(a.astype(np.float32))) if dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    x = cast(2.0 * rng.standard_normal((B, d)))
    w = cast(1.0 + 0.1 * rng.standard_normal(d))
    table = cast(rng.standard_normal((V, emb_dim))) if emb_dim else None
    return x, w, table


def _bits(t, dtype):
    torch = torch_mod()
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy().view(np.uint32)


def _np_bits(a, dtype):
    return a.view(np.uint16) if dtype == "bf16" else np.asarray(a, np.float32).view(np.uint32)


def _check(head, w, x, nw, table, eps, normalizer, K):
    torch = torch_mod()
    B = x.shape[0]
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    h, tok, emb = head.draft_step(to_device(x, w.dtype), to_device(nw, w.dtype), eps, K,
                                  None if table is None else to_device(table, w.dtype),
                                  normalizer, topk_out=tk)
    torch.cuda.synchronize()
    h_o, tok_o, emb_o, sel_o = od.draft_step(x, nw, eps, w.C, w.E, w.offsets, w.tos, K, table,
                                             normalizer, w.dtype)
    assert np.array_equal(_bits(h, w.dtype), _np_bits(h_o, w.dtype))
    assert tk.cpu().numpy().tolist() == sel_o.tolist()
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    if table is None:
        assert emb is None
    else:
        assert np.array_equal(_bits(emb, w.dtype), _np_bits(emb_o, w.dtype))


@pytest.mark.parametrize("K,B", [(4, 3), (64, 4)])
def test_tiny_config_f32(K, B):
    w = make_workload("tiny")
    x, nw, table = _inputs(1, B, w.d, w.V, 12, "f32")
    _check(make_head(w, max_B=4), w, x, nw, table, 1e-6, 2.5, K)


@pytest.mark.parametrize("seed,d,V,Nc,K,B,emb_dim,ragged", [
    (51, 128, 8192, 64, 4, 9, 64, False),
    (52, 64, 3000, 40, 3, 7, 40, True),      # ragged clusters, some tiny
    (53, 256, 16384, 256, 16, 64, 2560, False),
    (54, 320, 5000, 50, 2, 70, 8, True),     # two passes of rows, d not a multiple of 256
    (55, 192, 4096, 64, 5, 5, 0, False),     # no embedding table
])
def test_random_shapes(seed, d, V, Nc, K, B, emb_dim, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    x, nw, table = _inputs(seed, B, d, V, emb_dim, "bf16")
    _check(make_head(w, max_B=B), w, x, nw, table, 1e-6, float(np.sqrt(2560.0)), K)


def test_sweep_config_full_size():
    """The sweep head (d=256, V=262144, Nc=2048, K=32, bf16) at B=64 as the
    bench runs it: every normalised row and token against the oracle."""
    w = make_workload("sweep")
    x, nw, table = _inputs(60, 64, w.d, w.V, 128, "bf16")
    _check(make_head(w, max_B=64), w, x, nw, table, 1e-6, float(np.sqrt(2560.0)), w.K)


def test_sum_of_squares_in_element_order():
    """The absorbed-squares row of tests/golden/draft_step.json on a float32
    head, with the oracle's value and the hand-derived bits: the outputs are
    0x33c00002 only when the squares are summed in element order (a pairwise
    or any other order keeps some of the small squares and gives 0x33c00001).
    The norm's arithmetic is one template for both element types, so this
    pins the order of the bf16 heads' chain as well."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "draft_step.json")))
    case = next(c for c in gold["rms_norm"] if c["name"] == "absorbed_squares_f32")
    d = case["d"]
    x = np.full(d, int(case["x_rest"], 16), dtype=np.uint32)
    x[0] = int(case["x"]["0"], 16)
    nw = np.full(d, int(case["w_rest"], 16), dtype=np.uint32)
    nw[0] = int(case["w"]["0"], 16)
    want = np.full(d, int(case["expect_rest"], 16), dtype=np.uint32)
    want[0] = int(case["expect"]["0"], 16)
    w = make_random(61, d=d, V=1024, Nc=16, dtype="f32", rows=64, ragged=False)
    # the row three times (by itself, and between random rows), so that the
    # chain runs in rows of every position of a pass
    xs = np.stack([x.view(np.float32)] * 3)
    xs[1] = np.random.default_rng(5).standard_normal(d).astype(np.float32)
    head = make_head(w, max_B=3)
    h, _, _ = head.draft_step(to_device(xs, "f32"), to_device(nw.view(np.float32), "f32"),
                              float(case["eps"]) or 1e-30, 4)
    torch_mod().cuda.synchronize()
    got = _bits(h, "f32")
    assert np.array_equal(got[0], want) and np.array_equal(got[2], want)
    h_o = od.rms_norm(xs, nw.view(np.float32), float(case["eps"]) or 1e-30, "f32")
    assert np.array_equal(got, _np_bits(h_o, "f32"))


def test_zero_rows_large_eps_and_identity_scale():
    """A zero row normalises to signed zeros; eps = 4 dominates; normalizer 1
    returns the table rows unchanged."""
    w = make_random(56, d=128, V=4096, Nc=32, dtype="bf16", rows=64, ragged=False)
    x, nw, table = _inputs(56, 6, 128, 4096, 16, "bf16")
    x[2] = 0
    x[4] = 0x8000   # -0 everywhere
    _check(make_head(w, max_B=6), w, x, nw, table, 4.0, 1.0, 4)


def test_empty_clusters_embed_zeros():
    """A row whose selected clusters own no token gets token -1 and a zero
    embedding."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    d = 64
    x = np.zeros((2, d), dtype=np.float32)
    x[0, 0] = 3.0
    x[1, 0] = -3.0
    C = np.zeros((4, d), dtype=np.float32)
    C[:, 0] = [5.0, 4.0, -1.0, -2.0]       # row 0 picks clusters 0,1 (empty)
    E = np.random.default_rng(0).standard_normal((128, d)).astype(np.float32)
    off = np.array([0, 0, 0, 100, 128], dtype=np.int32)
    tos = np.random.default_rng(1).permutation(128).astype(np.int32)
    nw = np.ones(d, dtype=np.float32)
    table = np.random.default_rng(2).standard_normal((128, 4)).astype(np.float32)
    head = Head(torch.from_numpy(C).cuda(), torch.from_numpy(E).cuda(), tos, off, max_B=2, max_K=4)
    h, tok, emb = head.draft_step(torch.from_numpy(x).cuda(), torch.from_numpy(nw).cuda(), 1e-6, 2,
                                  torch.from_numpy(table).cuda(), 3.0)
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    assert tok[0] == -1 and tok[1] >= 0
    e = emb.cpu().numpy()
    assert not e[0].any()
    assert np.array_equal(e[1], (table[tok[1]] * np.float32(3.0)).astype(np.float32))


def test_draft_step_errors():
    import ctypes
    from centroid_masked_sparse_amd import _ffi
    torch = torch_mod()
    w = make_workload("tiny")
    head = make_head(w, max_B=4)
    x, nw, table = _inputs(3, 2, w.d, w.V, 12, "f32")
    xd, nwd = to_device(x, "f32"), to_device(nw, "f32")
    td = to_device(table, "f32")
    lib = head._lib
    ws = head.new_workspace(2, 4, _ffi.CE_OP_DRAFT_STEP)
    hout = torch.empty_like(xd)
    tok = torch.empty(2, dtype=torch.int32, device="cuda:0")
    emb = torch.empty((2, 12), dtype=torch.float32, device="cuda:0")

    def call(x_ptr=xd.data_ptr(), nw_ptr=nwd.data_ptr(), eps=1e-6, h_ptr=hout.data_ptr(),
             t_ptr=td.data_ptr(), emb_dim=12, norm=1.0, e_ptr=emb.data_ptr()):
        return lib.ce_draft_step(head._handle, x_ptr, nw_ptr, ctypes.c_float(eps), 2, 4, h_ptr,
                                 tok.data_ptr(), t_ptr, emb_dim, ctypes.c_float(norm), e_ptr, None,
                                 ws.data_ptr(), ws.numel(), None)

    assert call(eps=0.0) == 2
    assert call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    assert call(emb_dim=3) == 2                 # 12-byte rows
    assert call(norm=float("inf")) == 2
    assert call(nw_ptr=None) == 1
    assert call(h_ptr=None) == 1
    assert call(e_ptr=None) == 1
    assert call(h_ptr=xd.data_ptr()) == 9       # in place: x and h_out overlap
    assert call(nw_ptr=nwd.data_ptr() + 4) == 4
    assert call(t_ptr=None, e_ptr=None) == 0    # no table: tokens only
    assert call() == 0
    torch.cuda.synchronize()


def test_draft_step_under_stream_capture():
    """ce_draft_step is capture-safe: a graph captured around it replays to
    the eager result, with other eager work and synchronisation between
    replays."""
    torch = torch_mod()
    w = make_random(57, d=256, V=8192, Nc=64, dtype="bf16", rows=16)
    head = make_head(w, max_B=16)
    x, nw, table = _inputs(57, 16, 256, 8192, 64, "bf16")
    xd, nwd, td = to_device(x, "bf16"), to_device(nw, "bf16"), to_device(table, "bf16")
    h_e, tok_e, emb_e = [t.clone() for t in head.draft_step(xd, nwd, 1e-6, 4, td, 3.0)]
    h = torch.empty_like(xd)
    tok = torch.empty(16, dtype=torch.int32, device="cuda:0")
    emb = torch.empty((16, 64), dtype=torch.bfloat16, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        head.draft_step(xd, nwd, 1e-6, 4, td, 3.0, h_out=h, out=tok, emb_out=emb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        head.draft_step(xd, nwd, 1e-6, 4, td, 3.0, h_out=h, out=tok, emb_out=emb)
    for _ in range(3):
        h.zero_()
        tok.fill_(-5)
        emb.fill_(7.0)
        head.top_tokens(h_e, 4)          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), h_e.view(torch.int16))
        assert torch.equal(tok, tok_e)
        assert torch.equal(emb.view(torch.int16), emb_e.view(torch.int16))
