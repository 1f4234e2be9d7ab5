"""GPU parity at the size limits of the boundary: the largest hidden size
(d = 8192, where every kernel takes its generic chunk loop and the fp32
draft step stages 64 KiB of normalised rows in LDS), the largest centroid
count (Nc = 8192) with K = Nc, batches of several 64-row passes, and a
vocabulary of 2^23 tokens."""

import numpy as np
import pytest

import oracle
from oracle import draft as od
from oracle import fp8_slabs as f8
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random
from workloads.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _bits(t, dtype):
    torch = torch_mod()
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy().view(np.uint32)


def _np_bits(a, dtype):
    return a.view(np.uint16) if dtype == "bf16" else np.asarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("dtype,V,Nc,K,B", [("bf16", 2048, 8, 2, 3), ("f32", 1024, 4, 2, 2)])
def test_largest_hidden_size(dtype, V, Nc, K, B):
    torch = torch_mod()
    d = 8192
    w = make_random(71, d=d, V=V, Nc=Nc, dtype=dtype, rows=8)
    head = make_head(w, max_B=B)
    hb = rows(w, B)
    h = to_device(hb, dtype)
    tok = head.top_tokens(h, K)
    masked = head.masked_logits(h, K)
    tm, vm = head.top_m(h, 8, K)
    torch.cuda.synchronize()
    tok_o, sel_o, _ = oracle.top_tokens(hb, w.C, w.E, w.offsets, w.tos, K, dtype)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    M, _ = oracle.masked_logits(hb, w.C, w.E, w.offsets, w.tos, K, dtype)
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
    tm_o, vm_o = oracle.top_m(hb, w.C, w.E, w.offsets, w.tos, K, 8, dtype)
    assert tm.cpu().numpy().tolist() == tm_o.tolist()
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), vm_o.view(np.uint32))
    # the draft step at d = 8192
    rng = np.random.default_rng(71)
    cast = (lambda a: f32_to_bf16_bits(a.astype(np.float32))) if dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    x = cast(2.0 * rng.standard_normal((B, d)))
    nw = cast(1.0 + 0.1 * rng.standard_normal(d))
    table = cast(rng.standard_normal((V, 32)))
    hn, tk, emb = head.draft_step(to_device(x, dtype), to_device(nw, dtype), 1e-6, K,
                                  to_device(table, dtype), 3.0)
    torch.cuda.synchronize()
    h_o, tok_d, emb_o, _ = od.draft_step(x, nw, 1e-6, w.C, w.E, w.offsets, w.tos, K, table, 3.0,
                                         dtype)
    assert np.array_equal(_bits(hn, dtype), _np_bits(h_o, dtype))
    assert tk.cpu().numpy().tolist() == tok_d.tolist()
    assert np.array_equal(_bits(emb, dtype), _np_bits(emb_o, dtype))


def test_largest_hidden_size_fp8():
    from centroid_masked_sparse_amd import Head
    torch = torch_mod()
    w = make_random(72, d=8192, V=2048, Nc=8, dtype="bf16", rows=4)
    head = Head(to_device(w.C, "bf16"), to_device(w.E, "bf16"), w.tos, max_B=3, max_K=8, slabs="fp8")
    hb = rows(w, 3)
    tok = head.top_tokens(to_device(hb, "bf16"), 2)
    torch.cuda.synchronize()
    codes, sc = f8.quantize_rows(w.E)
    tok_o, _ = f8.top_tokens_fp8(hb, w.C, codes, sc, w.offsets, w.tos, 2)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()


def test_largest_centroid_count_take_all():
    """Nc = 8192 centroids of one token each; K = Nc keeps every centroid, so
    the argmax is the dense argmax over all V tokens."""
    torch = torch_mod()
    w = make_random(73, d=64, V=8192, Nc=8192, dtype="bf16", rows=4)
    head = make_head(w, max_B=2)
    hb = rows(w, 2)
    tk = torch.full((2, 8192), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(to_device(hb, "bf16"), 8192, topk_out=tk)
    tok_small = head.top_tokens(to_device(hb, "bf16"), 300)
    torch.cuda.synchronize()
    assert tk.cpu().numpy().tolist() == [list(range(8192))] * 2
    dense = oracle.dense_logits(hb, w.E, w.tos, "bf16")
    want = [int(np.flatnonzero(r == r.max()).min()) for r in dense]
    assert tok.cpu().numpy().tolist() == want
    tok_o, _, _ = oracle.top_tokens(hb, w.C, w.E, w.offsets, w.tos, 300, "bf16")
    assert tok_small.cpu().numpy().tolist() == tok_o.tolist()


def test_three_passes_of_rows():
    """B = 150: passes of 64, 64 and 22 rows; every row equals the oracle and
    does not depend on the batch it came in."""
    torch = torch_mod()
    w = make_random(74, d=128, V=4096, Nc=64, dtype="bf16", rows=64)
    head = make_head(w, max_B=150)
    hb = rows(w, 150)
    tok = head.top_tokens(to_device(hb, "bf16"), 5)
    torch.cuda.synchronize()
    tok_o, _, _ = oracle.top_tokens(hb[:64], w.C, w.E, w.offsets, w.tos, 5, "bf16")
    got = tok.cpu().numpy()
    assert got[:64].tolist() == tok_o.tolist()
    assert got[64:128].tolist() == tok_o.tolist() and got[128:].tolist() == tok_o[:22].tolist()


@pytest.mark.parametrize("B", [2, 6])
def test_largest_vocabulary(B):
    """A vocabulary of 2^23 tokens (d = 64, Nc = 8192 clusters of 1024, 16
    tiles each, 131072 tiles in all): token ids, tile indices and the
    forward's row offsets all pass 2^22.  B = 2 runs the by-row gather, B = 6
    the tile grid.  The bf16 values are drawn directly as bit patterns (one
    seeded integer draw: random sign and mantissa, exponents 2^-7 .. 2^0),
    which keeps the 8M x 64 draw to seconds."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    d, V, Nc, K = 64, 1 << 23, 8192, 4
    rng = np.random.default_rng(77)

    def bf16_bits(n):
        r = np.frombuffer(rng.bytes(2 * n), dtype=np.uint16)
        exp = (np.uint16(120) + ((r >> np.uint16(7)) & np.uint16(7))) << np.uint16(7)
        return (r & np.uint16(0x807F)) | exp

    E = bf16_bits(V * d).reshape(V, d)
    C = bf16_bits(Nc * d).reshape(Nc, d)
    h = bf16_bits(B * d).reshape(B, d)
    tos = rng.permutation(V).astype(np.int32)
    offsets = (np.arange(Nc + 1) * (V // Nc)).astype(np.int32)
    head = Head(to_device(C, "bf16"), to_device(E, "bf16"), tos, max_B=B, max_K=K)
    hd = to_device(h, "bf16")
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(hd, K, topk_out=tk)
    masked = head.masked_logits(hd, K)
    torch.cuda.synchronize()
    tok_o, sel_o, _ = oracle.top_tokens(h, C, E, offsets, tos, K, "bf16")
    assert tk.cpu().numpy().tolist() == sel_o.tolist()
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    M, _ = oracle.masked_logits(h, C, E, offsets, tos, K, "bf16")
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
    head.close()
