"""Seeded synthetic workloads for the centroid-masked sparse LM head.

The real assistant checkpoints (trained centroids, token ordering, embedding
table) are not available, so every workload here is drawn from a seeded
``numpy.random.default_rng`` (PCG64) stream with the shapes, dtypes and value
scales of the five benchmark workloads, named:

* ``tiny``    d=64,   V=4096,   Nc=64,   K=4 (also K=64), all fp32, h,C,E ~ N(0,1/d)
* ``sweep``   d=256,  V=262144, Nc=2048, K=32, bf16, h ~ N(0,1), C,E ~ N(0,1/d)
* ``masked``  the arrays of ``sweep`` (same seed), run at B in {1,16,64}
* ``wide``    d=1024, V=262144, Nc=4096, K=64 (also K=4096), bf16, as ``sweep``
* ``skewed``  d=512,  V=262144, Nc=2048, K=32, bf16, Zipf(1.1) cluster sizes,
              rows drawn around 8 anchor centroid directions

Recipe (fixed, so that any implementation can regenerate the bytes):

* ``rng = default_rng(seed)``; draws happen in this order: ``tos`` (a random
  permutation of the V token ids: ``tos[j]`` is the token stored at slot j of
  the ordered layout), then for ``skewed`` the rank->cluster permutation, the
  8 anchor centroids and the 64 row groups, then C, then E (drawn directly in
  the ordered layout, in chunks of whole rows), then h.
* Normals are float64 ``standard_normal`` draws times the standard deviation
  (N(0, v) means variance v), rounded to fp32 (round-to-nearest-even) and, for
  bf16 workloads, to bf16 by round-to-nearest-even of the fp32 value.
* 64 hidden rows are drawn for every workload; a batch of B rows is the first
  B of them, so results for row b must not depend on B.

bf16 arrays are stored as ``uint16`` bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache

import numpy as np

MAX_ROWS = 64
_CHUNK_ELEMS = 1 << 24


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    seed: int
    d: int
    V: int
    Nc: int
    K: int
    dtype: str            # "f32" or "bf16": element type of h, C and E
    h_dist: str           # "inv_d": N(0,1/d); "unit": N(0,1); "anchored": see module doc
    batches: tuple        # batch sizes the configuration is run at
    extra_K: tuple = ()   # further K values run on the same arrays
    zipf_s: float | None = None
    anchors: int = 0
    noise_var: float = 0.0


CONFIGS = {
    "tiny": ConfigSpec("tiny", 1, 64, 4096, 64, 4, "f32", "inv_d", (1,), (64,)),
    "sweep": ConfigSpec("sweep", 2, 256, 262144, 2048, 32, "bf16", "unit",
                        (1, 2, 4, 8, 16, 32, 64)),
    "masked": ConfigSpec("masked", 2, 256, 262144, 2048, 32, "bf16", "unit",
                         (1, 16, 64)),
    "wide": ConfigSpec("wide", 4, 1024, 262144, 4096, 64, "bf16", "unit",
                       (64,), (4096,)),
    "skewed": ConfigSpec("skewed", 5, 512, 262144, 2048, 32, "bf16", "anchored",
                         (64,), (), zipf_s=1.1, anchors=8, noise_var=0.1),
}


@dataclass
class Workload:
    """One drawn workload.  Arrays are host numpy arrays."""

    name: str
    seed: int
    d: int
    V: int
    Nc: int
    K: int
    dtype: str
    h: np.ndarray          # [64, d]  float32, or uint16 bf16 bits
    C: np.ndarray          # [Nc, d]  centroid rows
    E: np.ndarray          # [V, d]   embeddings in the ordered (slot) layout
    offsets: np.ndarray    # [Nc+1] int32: cluster c owns slots [offsets[c], offsets[c+1])
    tos: np.ndarray        # [V] int32: token id stored at each slot
    groups: np.ndarray | None = None   # skewed: anchor group of each row
    anchor_ids: np.ndarray | None = None

    @property
    def sizes(self) -> np.ndarray:
        return np.diff(self.offsets.astype(np.int64))


def f32_to_bf16_bits(x: np.ndarray, out: np.ndarray | None = None,
                     tmp: np.ndarray | None = None) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Works in uint32: for finite inputs ``bits + 0x7FFF + lsb`` cannot wrap.
    ``out`` (uint16) and ``tmp`` (uint32) may be passed to avoid allocations.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in synthetic data")
    b = x.view(np.uint32)
    if tmp is None:
        tmp = np.empty(b.shape, dtype=np.uint32)
    np.right_shift(b, 16, out=tmp)
    np.bitwise_and(tmp, 1, out=tmp)
    tmp += 0x7FFF
    tmp += b
    tmp >>= 16
    if out is None:
        return tmp.astype(np.uint16)
    out[...] = tmp
    return out


def _bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _normal_rows(rng, n: int, d: int, std: float, dtype: str) -> np.ndarray:
    out = np.empty((n, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    rows = max(1, min(n, _CHUNK_ELEMS // d))
    buf64 = np.empty((rows, d), dtype=np.float64)   # reused: first touch is costly
    buf32 = np.empty((rows, d), dtype=np.float32)
    tmp = np.empty((rows, d), dtype=np.uint32)
    for r0 in range(0, n, rows):
        m = min(n, r0 + rows) - r0
        rng.standard_normal(out=buf64[:m])
        buf64[:m] *= std
        buf32[:m] = buf64[:m]                        # float64 -> fp32, nearest-even
        if dtype == "f32":
            out[r0:r0 + m] = buf32[:m]
        else:
            f32_to_bf16_bits(buf32[:m], out=out[r0:r0 + m], tmp=tmp[:m])
    return out


def zipf_sizes(Nc: int, V: int, s: float, rank_to_cluster: np.ndarray) -> np.ndarray:
    """Cluster sizes following Zipf(s) over ranks, summing exactly to V.

    Rank r (1-based) gets ``max(1, floor(V * r**-s / H))`` with
    ``H = sum_r r**-s``; the remainder ``V - sum`` adds one token to each of the
    first ``remainder`` ranks.  Rank r is cluster ``rank_to_cluster[r-1]``.
    """
    r = np.arange(1, Nc + 1, dtype=np.float64)
    w = r ** (-s)
    n = np.maximum(1, np.floor(V * w / w.sum())).astype(np.int64)
    rem = V - int(n.sum())
    if rem < 0 or rem > Nc:
        raise ValueError("Zipf sizes cannot be balanced to V")
    n[:rem] += 1
    sizes = np.empty(Nc, dtype=np.int64)
    sizes[rank_to_cluster] = n
    return sizes


def _offsets_from_sizes(sizes: np.ndarray) -> np.ndarray:
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=off[1:])
    return off.astype(np.int32)


@lru_cache(maxsize=4)
def make_workload(name: str) -> Workload:
    """Draw the workload called ``name`` (a key of CONFIGS); ``masked`` shares
    the arrays of ``sweep``."""
    spec = CONFIGS[name]
    if name == "masked":
        w = make_workload("sweep")
        return Workload(spec.name, w.seed, w.d, w.V, w.Nc, spec.K, w.dtype, w.h, w.C,
                        w.E, w.offsets, w.tos)
    rng = np.random.default_rng(spec.seed)
    d, V, Nc = spec.d, spec.V, spec.Nc
    tos = rng.permutation(V).astype(np.int32)
    groups = anchor_ids = None
    if spec.zipf_s is not None:
        sigma = rng.permutation(Nc)
        anchor_ids = rng.choice(Nc, size=spec.anchors, replace=False)
        groups = rng.integers(0, spec.anchors, size=MAX_ROWS)
        offsets = _offsets_from_sizes(zipf_sizes(Nc, V, spec.zipf_s, sigma))
    else:
        if V % Nc:
            raise ValueError("equal clusters need V % Nc == 0")
        offsets = (np.arange(Nc + 1, dtype=np.int64) * (V // Nc)).astype(np.int32)
    w_std = 1.0 / np.sqrt(d)
    C = _normal_rows(rng, Nc, d, w_std, spec.dtype)
    E = _normal_rows(rng, V, d, w_std, spec.dtype)
    if spec.h_dist == "anchored":
        Cf = C.astype(np.float64) if spec.dtype == "f32" else _bf16_bits_to_f64(C)
        dirs = Cf[anchor_ids[groups]]
        dirs = dirs / np.linalg.norm(dirs, axis=1, keepdims=True) * np.sqrt(d)
        noise = rng.standard_normal((MAX_ROWS, d)) * np.sqrt(spec.noise_var)
        h = _cast(dirs + noise, spec.dtype)
    else:
        h_std = 1.0 if spec.h_dist == "unit" else w_std
        h = _normal_rows(rng, MAX_ROWS, d, h_std, spec.dtype)
    return Workload(spec.name, spec.seed, d, V, Nc, spec.K, spec.dtype, h, C, E,
                    offsets, tos, groups, anchor_ids)


def make_random(seed: int, d: int, V: int, Nc: int, dtype: str = "bf16",
                rows: int = MAX_ROWS, K: int = 4, ragged: bool = False,
                h_std: float = 1.0) -> Workload:
    """A small random workload for edge-case tests.

    With ``ragged`` the cluster sizes are a random composition of V into Nc
    parts (cut points drawn uniformly with replacement), so some clusters may
    be empty; otherwise V % Nc must be 0 and all clusters are equal.
    """
    rng = np.random.default_rng(seed)
    tos = rng.permutation(V).astype(np.int32)
    if ragged:
        cuts = np.sort(rng.integers(0, V + 1, size=Nc - 1))
        offsets = np.concatenate([[0], cuts, [V]]).astype(np.int32)
    else:
        if V % Nc:
            raise ValueError("equal clusters need V % Nc == 0")
        offsets = (np.arange(Nc + 1, dtype=np.int64) * (V // Nc)).astype(np.int32)
    w_std = 1.0 / np.sqrt(d)
    C = _normal_rows(rng, Nc, d, w_std, dtype)
    E = _normal_rows(rng, V, d, w_std, dtype)
    h = _normal_rows(rng, rows, d, h_std, dtype)
    return Workload(f"random{seed}", seed, d, V, Nc, K, dtype, h, C, E, offsets, tos)
