"""GPU parity of the gather's two launch shapes.

With equal clusters the float64 gather launches one wave per selected (row,
centroid, tile), reading the centroid from the row's top-K ids, for batches
of up to 4 rows, and up to 47 rows while B*K <= 2*Nc (FP8 argmax: at every
batch); otherwise one wave per tile of the head (two per tile from 48 rows),
reading the rows that selected it from the selection words.  Both must give
every row the oracle's answer, including rows that select the same clusters
(identical rows: by row, two waves then dot the same tile).  The batch sizes
below reach both shapes on each head and both sides of the B*K = 2*Nc edge
(head 82: 42 rows by row, 43 on the tile grid; head 83: 32 by row, 40 on
the tile grid).
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,d,V,Nc,K", [
    (81, 128, 4096, 64, 5),     # one tile per cluster
    (82, 64, 8192, 64, 3),      # two tiles per cluster
    (83, 256, 16384, 256, 16),
])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 30, 32, 40, 42, 43, 47, 48])
def test_by_row_and_tile_grid_agree_with_oracle(seed, d, V, Nc, K, B):
    torch = torch_mod()
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=False)
    hb = rows(w, B).copy()
    if B >= 2:
        hb[1] = hb[0]          # duplicate selections
    if B >= 4:
        hb[3] = hb[0]
    head = make_head(w, max_B=64)
    h = to_device(hb, "bf16")
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(h, K, topk_out=tk)
    masked = head.masked_logits(h, K)
    tm, vm = head.top_m(h, 6, K)
    torch.cuda.synchronize()
    tok_o, sel_o, _ = oracle.top_tokens(hb, w.C, w.E, w.offsets, w.tos, K, "bf16")
    assert tk.cpu().numpy().tolist() == sel_o.tolist()
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    M, _ = oracle.masked_logits(hb, w.C, w.E, w.offsets, w.tos, K, "bf16")
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
    tm_o, vm_o = oracle.top_m(hb, w.C, w.E, w.offsets, w.tos, K, 6, "bf16")
    assert tm.cpu().numpy().tolist() == tm_o.tolist()
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), vm_o.view(np.uint32))


@pytest.mark.parametrize("B", [1, 2, 4, 5])
def test_by_row_and_tile_grid_fp8(B):
    """The same two launch shapes on FP8 slabs (bf16 rows, E4M3 codes with
    row scales): tokens and masked rows equal the FP8 oracle's."""
    from centroid_masked_sparse_amd import Head
    from oracle import fp8_slabs as f8
    torch = torch_mod()
    w = make_random(84, d=128, V=8192, Nc=64, dtype="bf16", rows=64, ragged=False)
    hb = rows(w, B).copy()
    if B >= 2:
        hb[1] = hb[0]
    head = Head(to_device(w.C, "bf16"), to_device(w.E, "bf16"), w.tos, max_B=8, max_K=8, slabs="fp8")
    h = to_device(hb, "bf16")
    tok = head.top_tokens(h, 4)
    masked = head.masked_logits(h, 4)
    torch.cuda.synchronize()
    codes, sc = f8.quantize_rows(w.E)
    tok_o, _ = f8.top_tokens_fp8(hb, w.C, codes, sc, w.offsets, w.tos, 4)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    M = f8.masked_logits_fp8(hb, w.C, codes, sc, w.offsets, w.tos, 4)
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
