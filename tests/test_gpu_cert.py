"""GPU parity of the certified matrix-core argmax (projection="mfma" forces
it on every tile-grid call of a bf16 head) against the oracle.

The gather bounds each matrix-core sum and the finalize recomputes canonical
keys only where the bounds leave the winner open, so the tokens must equal
the oracle's bit for bit on every path of the finalize: a single token that
alone reaches the best lower bound, named tokens recomputed by waves, whole
tiles recomputed a lane per slot, and whole rows (tied logits, zero rows).
"""

import dataclasses

import numpy as np
import pytest

import oracle
from oracle import fp8_slabs as f8
from tests.gpu_helpers import make_head, rows, to_device, torch_mod
from workloads import make_random

pytestmark = pytest.mark.gpu


def _fp8_head(w, max_B, max_K):
    from centroid_masked_sparse_amd import Head
    equal = np.all(np.diff(w.offsets) == w.V // w.Nc) and w.V % w.Nc == 0
    return Head(to_device(w.C, w.dtype), to_device(w.E, w.dtype), w.tos,
                None if equal else w.offsets, max_B=max_B, max_K=max_K, slabs="fp8",
                projection="mfma")


def _tokens(head, w, B, K):
    torch = torch_mod()
    tk = torch.full((B, K), -7, dtype=torch.int32, device="cuda:0")
    tok = head.top_tokens(to_device(rows(w, B), w.dtype), K, topk_out=tk)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), tk.cpu().numpy()


@pytest.mark.parametrize("seed,d,V,Nc,K,B,ragged", [
    (201, 64, 8192, 64, 4, 5, False),       # smallest tile-grid batch
    (202, 128, 20000, 100, 6, 16, True),     # ragged: shared tiles, tiny clusters
    (203, 256, 16384, 128, 8, 64, False),
    (204, 512, 12000, 90, 5, 64, True),      # many rows per tile: several passes
    (205, 320, 8192, 64, 3, 70, False),      # generic pipeline, two passes of rows
    (206, 1024, 8192, 128, 16, 33, False),
])
def test_bf16_heads(seed, d, V, Nc, K, B, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    head = make_head(w, max_B=B, max_K=K, projection="mfma")
    tok, tk = _tokens(head, w, B, K)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()


@pytest.mark.parametrize("seed,d,V,Nc,K,B,ragged", [
    (211, 128, 8192, 64, 4, 9, False),
    (212, 64, 3000, 40, 3, 17, True),
    (213, 512, 5000, 50, 2, 70, True),
])
def test_fp8_heads(seed, d, V, Nc, K, B, ragged):
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    head = _fp8_head(w, max_B=B, max_K=K)
    tok, tk = _tokens(head, w, B, K)
    codes, sc = f8.quantize_rows(w.E)
    tok_o, sel_o = f8.top_tokens_fp8(rows(w, B), w.C, codes, sc, w.offsets, w.tos, K)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()


@pytest.mark.parametrize("ragged,K", [(False, 4), (True, 4), (False, 32), (False, 48)])
def test_near_ties_and_exact_ties(ragged, K):
    """Embedding rows drawn from a pool of 4, half of them nudged by one bf16
    ulp in one dim: every row's best logit is shared by many tokens (whole
    tiles and whole rows recomputed) or missed by a hair (named tokens
    recomputed); a zero row ties every candidate at +0.  K = 32 and 48 put
    32 and 48 rows on each selected tile of the equal clusters: passes of
    two and four row groups."""
    w = make_random(221, d=128, V=16384, Nc=64, dtype="bf16", rows=64, ragged=ragged)
    rng = np.random.default_rng(222)
    P = w.E[rng.integers(0, w.V, size=4)]
    E = np.ascontiguousarray(P[rng.integers(0, 4, size=w.V)])
    nudge = rng.random(w.V) < 0.5
    E[nudge, 7] = E[nudge, 7] + 1            # next bf16 bit pattern: one ulp away
    h = w.h.copy()
    h[3] = 0
    w = dataclasses.replace(w, E=E, h=h)
    B = 64
    head = make_head(w, max_B=B, max_K=K, projection="mfma")
    tok, tk = _tokens(head, w, B, K)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()


@pytest.mark.parametrize("seed,d,V,Nc,K,B,fp8", [
    (251, 256, 8192, 64, 32, 64, False),     # 32 rows a tile: two row groups
    (252, 512, 6400, 50, 40, 64, False),     # 51: four row groups
    (253, 320, 4096, 32, 20, 40, False),     # 25, generic pipeline: two
    (254, 192, 4096, 16, 16, 70, False),     # K = Nc, 64 then 6 rows: four, then one
    (255, 256, 8192, 64, 48, 64, True),      # FP8 slabs, 48: four
    (256, 128, 4096, 32, 12, 50, True),      # FP8 slabs, 18: two
    (257, 1024, 8192, 128, 64, 64, False),   # 32 rows, d = 1024: two
    (258, 1024, 8192, 64, 64, 64, False),    # K = Nc, d = 1024: four
    (259, 320, 4096, 32, 30, 40, False),     # 37 rows of 40, generic pipeline: four
    (260, 2048, 2048, 16, 16, 64, False),    # d = 2048, past the rows-in-LDS limit: four
    (261, 1024, 2048, 32, 24, 64, True),     # FP8 slabs, d = 1024, 48: four
])
def test_row_groups(seed, d, V, Nc, K, B, fp8):
    """Equal clusters whose selected tiles carry more than 16 rows on
    average (B K / Nc): a pass takes two or four groups of 16 rows, each
    loaded block feeding every group's instructions; four groups run in the
    persistent kernel with the pass's rows in LDS up to d = 1024."""
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=max(64, B), ragged=False)
    head = _fp8_head(w, max_B=B, max_K=K) if fp8 else make_head(w, max_B=B, max_K=K, projection="mfma")
    tok, tk = _tokens(head, w, B, K)
    if fp8:
        codes, sc = f8.quantize_rows(w.E)
        tok_o, sel_o = f8.top_tokens_fp8(rows(w, B), w.C, codes, sc, w.offsets, w.tos, K)
    else:
        tok_o, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert tk.tolist() == sel_o.tolist()
    assert tok.tolist() == tok_o.tolist()


def test_exact_and_certified_agree_on_repeated_calls():
    """The records need no clearing: calls with different rows on one
    workspace give the oracle's tokens each time."""
    w = make_random(231, d=512, V=16384, Nc=128, dtype="bf16", rows=64, ragged=True)
    B, K = 24, 6
    head = make_head(w, max_B=64, max_K=K, projection="mfma")
    for lo in (0, 40, 17):
        hb = np.ascontiguousarray(w.h[lo:lo + B])
        tok = head.top_tokens(to_device(hb, w.dtype), K)
        tok_o, _, _ = oracle.top_tokens(hb, w.C, w.E, w.offsets, w.tos, K, w.dtype)
        assert tok.cpu().numpy().tolist() == tok_o.tolist(), lo


@pytest.mark.parametrize("ragged,B,K", [(False, 16, 5), (True, 64, 5), (False, 64, 40)])
def test_certified_argmax_graph_replays(ragged, B, K):
    """Captured once and replayed with eager work in between: the certified
    path's records are rewritten by each replay, so every replay gives the
    oracle's tokens.  K = 40 of 96 equal clusters puts 26 rows on each
    selected tile at B = 64: passes of two row groups."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    V = 12000 if ragged else 96 * 128
    w = make_random(241 + B + K, d=512, V=V, Nc=96, dtype="bf16", rows=64, ragged=ragged)
    head = make_head(w, max_B=64, max_K=K, projection="mfma")
    h = to_device(rows(w, B), w.dtype)
    out = torch.full((B,), -9, dtype=torch.int32, device="cuda:0")
    tk = torch.full((B, K), -9, dtype=torch.int32, device="cuda:0")
    g = head.capture(OP_TOP_TOKENS, h, K, out, topk_out=tk)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    other = to_device(np.ascontiguousarray(w.h[::-1][:B]), w.dtype)
    for i in range(4):
        out.fill_(-9)
        tk.fill_(-9)
        g.launch()
        torch.cuda.synchronize()
        assert out.cpu().tolist() == tok_o.tolist(), i
        assert tk.cpu().tolist() == sel_o.tolist(), i
        head.top_tokens(other, K)       # eager calls rewrite the records in between
        torch.cuda.synchronize()
    g.close()


def test_rows_in_lds_kernel_under_graph_replays():
    """The persistent certified gather (64 rows a pass, the rows in LDS)
    captured into a graph and replayed against the oracle, with eager calls
    of another batch in between."""
    torch = torch_mod()
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    w = make_random(262, d=256, V=8192, Nc=64, dtype="bf16", rows=64, ragged=False)
    B, K = 64, 48                          # 48 rows on each selected tile
    head = make_head(w, max_B=B, max_K=K, projection="mfma")
    h = to_device(rows(w, B), w.dtype)
    out = torch.full((B,), -9, dtype=torch.int32, device="cuda:0")
    g = head.capture(OP_TOP_TOKENS, h, K, out)
    tok_o, _, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    other = to_device(np.ascontiguousarray(w.h[::-1][:B]), w.dtype)
    for i in range(3):
        out.fill_(-9)
        g.launch()
        torch.cuda.synchronize()
        assert out.cpu().tolist() == tok_o.tolist(), i
        head.top_tokens(other, K)
        torch.cuda.synchronize()
    g.close()


def _random_case(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 192, 256, 512]))
    Nc = int(rng.integers(8, 160))
    V = int(rng.integers(Nc * 8, Nc * 96))
    ragged = bool(rng.random() < 0.6)
    K = int(rng.integers(1, min(Nc, 12) + 1))
    B = int(rng.choice([5, 9, 17, 33, 64, 65, 100]))
    fp8 = bool(rng.random() < 0.3)
    return d, V, Nc, K, B, ragged, fp8


@pytest.mark.parametrize("seed", range(300, 316))
def test_random_heads(seed):
    """Seeded random heads (equal or ragged clusters, d from 64 to 512, bf16
    or FP8 slabs, 5 to 100 rows) through the certified argmax."""
    d, V, Nc, K, B, ragged, fp8 = _random_case(seed)
    if not ragged:
        V = V // Nc * Nc
    w = make_random(seed, d=d, V=V, Nc=Nc, dtype="bf16", rows=64, ragged=ragged)
    head = _fp8_head(w, max_B=B, max_K=K) if fp8 else make_head(w, max_B=B, max_K=K, projection="mfma")
    tok, tk = _tokens(head, w, B, K)
    if fp8:
        codes, sc = f8.quantize_rows(w.E)
        tok_o, sel_o = f8.top_tokens_fp8(rows(w, B), w.C, codes, sc, w.offsets, w.tos, K)
    else:
        tok_o, sel_o, _ = oracle.top_tokens(rows(w, B), w.C, w.E, w.offsets, w.tos, K, w.dtype)
    assert tk.tolist() == sel_o.tolist(), (d, V, Nc, K, B, ragged, fp8)
    assert tok.tolist() == tok_o.tolist(), (d, V, Nc, K, B, ragged, fp8)
