"""The bf16-MFMA centroid projection and its certified top-K.

The fused calls of a bf16 head score the centroids with the matrix cores
(fp32 sums in an undocumented internal order) and certify the top-K against
an error bound E; near the K-th place they recompute canonical keys.  These
tests check, on the GPU:

* the error model the bound rests on: for every approximate score,
  |S~ - sum_k h_k C_ck| <= d 2^-23 sum_k |h_k C_ck| (each instruction adds 32
  exact products and the accumulator with at most 32 fp32 roundings or
  truncations), and the worst observed error over random and
  exponent-spread inputs is at most a quarter of that model;
* the whole bound E the top-K uses (Cauchy-Schwarz on the row norm and the
  largest centroid norm) holds for every score against the canonical key;
* selections and tokens equal the oracle's and the exact projection's,
  including rows whose boundary needs recomputed keys (constructed exact
  and near ties), rows recomputed whole (a zero row, fp32 overflow), and the
  counters that report both.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import rows, to_device, torch_mod
from workloads import make_random, make_workload
from workloads.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _head(w, projection, max_B=64, max_K=None):
    from centroid_masked_sparse_amd import Head
    equal = w.V % w.Nc == 0 and np.all(np.diff(w.offsets) == w.V // w.Nc)
    return Head(to_device(w.C, w.dtype), to_device(w.E, w.dtype), w.tos,
                None if equal else w.offsets, max_B=max_B,
                max_K=max_K if max_K is not None else w.Nc, projection=projection)


def _bf16_f64(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _spread(rng, n, d, lo, hi):
    """bf16 rows with every element's exponent drawn from [lo, hi]."""
    x = rng.standard_normal((n, d)) * np.exp2(rng.integers(lo, hi + 1, size=(n, d)))
    return f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("d,spread", [(256, 0), (256, 20), (512, 10), (1024, 0), (64, 30)])
def test_mfma_error_within_model(d, spread):
    torch = torch_mod()
    rng = np.random.default_rng(1000 + d + spread)
    Nc, B = 256, 64
    h = _spread(rng, B, d, -spread, spread) if spread else \
        f32_to_bf16_bits(rng.standard_normal((B, d)).astype(np.float32))
    C = _spread(rng, Nc, d, -spread - 4, spread - 4) if spread else \
        f32_to_bf16_bits((rng.standard_normal((Nc, d)) / np.sqrt(d)).astype(np.float32))
    w = make_random(7, d=d, V=Nc * 4, Nc=Nc, dtype="bf16", rows=4)
    import dataclasses
    w = dataclasses.replace(w, C=C)
    head = _head(w, "mfma")
    S = head.approx_scores(to_device(h, "bf16")).cpu().numpy().astype(np.float64)
    H, Cf = _bf16_f64(h), _bf16_f64(C)
    exact = H @ Cf.T                       # float64; off the exact sum by < d 2^-53 A
    A = np.abs(H) @ np.abs(Cf).T
    err = np.abs(S - exact)
    model = d * 2.0 ** -23 * A
    assert np.all(err <= model + d * 2.0 ** -125)
    nz = A > 0
    worst = float(np.max(err[nz] / A[nz]))
    # the model is at least four times the worst error seen
    assert 4 * worst <= d * 2.0 ** -23, worst / 2.0 ** -24
    # the top-K's bound E, with Cauchy-Schwarz and the largest centroid norm,
    # holds against the canonical keys themselves
    keys = oracle.centroid_scores(h, C, "bf16").astype(np.float64)
    cmax = np.sqrt((Cf * Cf).sum(axis=1)).max()
    Arow = np.sqrt((H * H).sum(axis=1)) * cmax
    beta = d * 2.0 ** -23
    E = beta * Arow * (1 + 2.0 ** -8) + 2.0 ** -23 * (np.abs(S).max(axis=1) + beta * Arow)
    assert np.all(np.abs(S - keys) <= E[:, None])


@pytest.mark.parametrize("name,Bs", [("sweep", (1, 2, 8, 64)), ("skewed", (64,))])
def test_projections_agree_with_oracle(name, Bs):
    """Both projections give the oracle's top-K ids and tokens, on the
    benchmark workloads."""
    torch = torch_mod()
    w = make_workload(name)
    tok_o, sel_o, _ = oracle.top_tokens(rows(w, 64), w.C, w.E, w.offsets, w.tos, w.K, w.dtype)
    for proj in ("mfma", "exact"):
        head = _head(w, proj)
        for B in Bs:
            tk = torch.full((B, w.K), -7, dtype=torch.int32, device="cuda:0")
            tok = head.top_tokens(to_device(rows(w, B), w.dtype), w.K, topk_out=tk)
            torch.cuda.synchronize()
            assert tk.cpu().tolist() == sel_o[:B].tolist(), (proj, B)
            assert tok.cpu().tolist() == tok_o[:B].tolist(), (proj, B)
        if proj == "mfma":
            print("repair counts", name, head.repair_counts())
        head.close()


def _near_tie_head(seed, Nc=64, d=128):
    """Centroids in pairs: (0, 1) equal, (2, 3) equal but for one element
    off by one bf16 step (keys a few ulps apart, far inside E), the rest
    random; rows aimed at those pairs, a zero row, and a row whose fp32 sums
    overflow."""
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((Nc, d)) / np.sqrt(d)
    C[1] = C[0]
    C[3] = C[2]
    C[5] = 1.0                                      # with row 3, a sum of 2^133
    Cb = f32_to_bf16_bits(C.astype(np.float32))
    Cb[3, 5] = Cb[2, 5] + 1                         # one bf16 step in one element
    V = Nc * 64
    E = f32_to_bf16_bits((rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32))
    tos = rng.permutation(V).astype(np.int32)
    h = rng.standard_normal((8, d))
    h[0] = 4 * C[0] + 0.01 * rng.standard_normal(d)   # pair (0, 1) near the top
    h[1] = 4 * C[2] + 0.01 * rng.standard_normal(d)
    h[2] = 0.0                                         # every score ties at 0
    hb = f32_to_bf16_bits(h.astype(np.float32))
    hb[3] = f32_to_bf16_bits(np.full(d, 2.0 ** 126, np.float32))  # fp32 sums overflow
    return Cb, E, tos, hb


@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_band_repair_and_whole_row_recompute(K):
    torch = torch_mod()
    from centroid_masked_sparse_amd import Head
    C, E, tos, h = _near_tie_head(11 + K)
    Nc = C.shape[0]
    off = np.arange(Nc + 1, dtype=np.int32) * 64
    hd = to_device(h, "bf16")
    res = {}
    for proj in ("mfma", "exact"):
        head = Head(to_device(C, "bf16"), to_device(E, "bf16"), tos, None, max_B=8, max_K=Nc,
                    projection=proj)
        tk = torch.full((8, K), -7, dtype=torch.int32, device="cuda:0")
        tok = head.top_tokens(hd, K, topk_out=tk)
        M = head.masked_logits(hd[:4], K)
        torch.cuda.synchronize()
        res[proj] = (tk.cpu().tolist(), tok.cpu().tolist(), M.cpu().numpy().view(np.uint32))
        if proj == "mfma":
            counts = head.repair_counts()
    tok_o, sel_o, _ = oracle.top_tokens(h, C, E, off, tos, K, "bf16")
    M_o, _ = oracle.masked_logits(h[:4], C, E, off, tos, K, "bf16")
    for proj in ("mfma", "exact"):
        assert res[proj][0] == sel_o.tolist(), proj
        assert res[proj][1] == tok_o.tolist(), proj
        assert np.array_equal(res[proj][2], M_o.view(np.uint32)), proj
    assert sel_o[2].tolist() == list(range(K))          # zero row: lowest ids
    # two calls of 8 and 4 rows: the zero row and the overflowing row are
    # recomputed whole in each (or take the band path, for the zero row when
    # the band fits); the tied pairs need their band recomputed
    assert counts[1] >= 2, counts
    assert counts[0] + counts[1] >= 4, counts


def test_approx_scores_rejects_fp32_heads():
    from centroid_masked_sparse_amd import CeError
    w = make_workload("tiny")
    head = _head(w, "auto")
    with pytest.raises(CeError) as e:
        head.approx_scores(to_device(rows(w, 1), w.dtype))
    assert e.value.status_name == "CE_ERR_BAD_DTYPE"
