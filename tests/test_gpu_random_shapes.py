"""GPU parity over seeded random shapes.

Each case draws a head (hidden size, vocabulary, centroid count, equal or
ragged clusters), a top-K and a batch size, so that together the cases pass
through every launch shape of the path: the by-row gather (up to 4 rows,
equal clusters), the tile grid, the split grid (48 rows or more), one- and
two-row projection waves, both projections (exact and the certified MFMA
one), and batches of several 64-row passes.  Tokens,
top-K ids, the forward rows and the top-m must equal the oracle's bit for
bit.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random

pytestmark = pytest.mark.gpu

_D = (64, 128, 192, 256, 320, 512)
_B = (1, 2, 3, 4, 5, 7, 8, 16, 31, 48, 64, 70)


def _case(i):
    r = np.random.default_rng(900 + i)
    d = int(r.choice(_D))
    Nc = int(r.choice([8, 16, 40, 64, 100, 128]))
    vpc = int(r.choice([16, 64, 70, 128, 200]))
    V = Nc * vpc
    ragged = bool(r.integers(2)) if i % 3 else False
    K = int(min(Nc, r.choice([1, 2, 3, 5, 8, 16, 32, 64])))
    B = int(_B[i % len(_B)])
    return d, V, Nc, K, B, ragged


@pytest.mark.parametrize("i", range(30))
def test_random_shape_against_oracle(i):
    torch = torch_mod()
    d, V, Nc, K, B, ragged = _case(i)
    w = make_random(900 + i, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    hb = rows(w, B)
    # odd cases take the certified MFMA projection, even ones the exact one
    head = make_head(w, max_B=B, projection="mfma" if i % 2 else "exact")
    h = to_device(hb, "bf16")
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(h, K, topk_out=tk)
    masked = head.masked_logits(h, K)
    m = 5
    tm, vm = head.top_m(h, m, K)
    torch.cuda.synchronize()
    tok_o, sel_o, _ = oracle.top_tokens(hb, w.C, w.E, w.offsets, w.tos, K, "bf16")
    assert tk.cpu().numpy().tolist() == sel_o.tolist(), (d, V, Nc, K, B, ragged)
    assert tok.cpu().numpy().tolist() == tok_o.tolist(), (d, V, Nc, K, B, ragged)
    M, _ = oracle.masked_logits(hb, w.C, w.E, w.offsets, w.tos, K, "bf16")
    assert np.array_equal(masked.cpu().numpy().view(np.uint32), M.view(np.uint32))
    tm_o, vm_o = oracle.top_m(hb, w.C, w.E, w.offsets, w.tos, K, m, "bf16")
    assert tm.cpu().numpy().tolist() == tm_o.tolist()
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), vm_o.view(np.uint32))
