"""Constructed ties on the GPU: equal logits across tiles, clusters and rows.

The pages' get_top_tokens takes the first maximum in candidate order; the
tie rule here (lowest token id, and for the top-m order logit descending then
token id ascending) makes the answer independent of that order, and these
tests build inputs where it decides: every embedding row is one of a few
distinct vectors, so each row's largest candidate logit is shared by a
hundred or more tokens spread over many tiles and clusters.  A zero hidden
row ties every centroid (top-K = the K lowest ids) and every logit (+0).
Each launch shape is covered: one wave per selected (row, centroid, tile) at
B <= 4, the tile grid, two waves per tile from 48 rows, and two passes of
rows.
"""

import dataclasses

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random

pytestmark = pytest.mark.gpu


def _pooled(seed, d, V, Nc, ragged, pool=6):
    """A random head whose ordered embedding rows are drawn from `pool`
    distinct rows; hidden row 1 is zero."""
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    rng = np.random.default_rng(seed + 1000)
    P = w.E[rng.integers(0, V, size=pool)]
    E = np.ascontiguousarray(P[rng.integers(0, pool, size=V)])
    h = w.h.copy()
    h[1] = 0
    return dataclasses.replace(w, E=E, h=h)


@pytest.mark.parametrize("proj", ["exact", "mfma"])
@pytest.mark.parametrize("ragged,B", [(False, 3), (False, 9), (False, 64), (False, 70),
                                      (True, 3), (True, 64)])
def test_tied_logits_tokens_top_m_and_rows(ragged, B, proj):
    torch = torch_mod()
    w = _pooled(81 + B, d=128, V=16384, Nc=128, ragged=ragged)   # 128 tokens (2 tiles) per cluster
    K, m = 6, 32
    head = make_head(w, max_B=B, max_K=K, projection=proj)
    hB = rows(w, B)
    h = to_device(hB, w.dtype)
    tok_o, sel_o, best_o = oracle.top_tokens(hB, w.C, w.E, w.offsets, w.tos, K, w.dtype)
    # the construction does tie: many candidates share each row's maximum
    for b in (0, 2, 3):
        b = b % B
        logits, tokens, _ = oracle.select_and_score(hB[b], w.C, w.E, w.offsets, w.tos, K, w.dtype)
        assert (logits == logits.max()).sum() >= 4, b
    assert sel_o[1].tolist() == list(range(K))                     # zero row: lowest ids

    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(h, K, topk_out=tk)
    tm, vm = head.top_m(h, m, K)
    M = head.masked_logits(h, K)
    torch.cuda.synchronize()
    assert tk.cpu().tolist() == sel_o.tolist()
    assert tok.cpu().tolist() == tok_o.tolist()
    tm_o, vm_o = oracle.top_m(hB, w.C, w.E, w.offsets, w.tos, K, m, w.dtype)
    assert tm.cpu().tolist() == tm_o.tolist()
    assert np.array_equal(vm.cpu().numpy().view(np.uint32), vm_o.view(np.uint32))
    M_o, _ = oracle.masked_logits(hB, w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert np.array_equal(M.cpu().numpy().view(np.uint32), M_o.view(np.uint32))


def _limit_head(m):
    """A ragged head whose largest cluster holds exactly 8160 - 64 m tiles of
    64 tokens (the most the top-m merge takes for a K = 1 selection), and two
    rows that select it."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    d, Nc = 64, 4
    big = (8160 - 64 * m) * 64
    sizes = np.array([big, 100, 60, 40])
    V = int(sizes.sum())
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rng = np.random.default_rng(91)
    from workloads.synth import f32_to_bf16_bits
    C = f32_to_bf16_bits((rng.standard_normal((Nc, d)) / 8).astype(np.float32))
    E = f32_to_bf16_bits((rng.standard_normal((V, d)) / 8).astype(np.float32))
    tos = rng.permutation(V).astype(np.int32)
    h = np.stack([C[0], C[0]]).copy()            # both rows point at centroid 0
    head = Head(to_device(C, "bf16"), to_device(E, "bf16"), tos, off, max_B=2, max_K=2)
    return head, h, C, E, off, tos


def test_top_m_at_the_merge_limit_and_one_past():
    torch = torch_mod()
    from centroid_masked_sparse_amd import CeError
    m = 8
    head, h, C, E, off, tos = _limit_head(m)
    hd = to_device(h, "bf16")
    tk = torch.full((2, 1), -7, dtype=torch.int32, device="cuda:0")
    tok, val = head.top_m(hd, m, 1, topk_out=tk)
    torch.cuda.synchronize()
    assert tk.cpu().tolist() == [[0], [0]]
    tok_o, val_o = oracle.top_m(h, C, E, off, tos, 1, m, "bf16")
    assert tok.cpu().tolist() == tok_o.tolist()
    assert np.array_equal(val.cpu().numpy().view(np.uint32), val_o.view(np.uint32))
    # one more output slot takes 64 more keys of LDS than the merge has
    with pytest.raises(CeError) as e:
        head.top_m(hd, m + 1, 1)
    assert e.value.status_name == "CE_ERR_UNSUPPORTED"
