"""Helpers for GPU tests: move seeded workloads to the device and build heads."""

from __future__ import annotations

import numpy as np


def torch_mod():
    import torch
    return torch


def to_device(a: np.ndarray, dtype: str):
    """numpy fp32 array or uint16 bf16 bits -> CUDA tensor of that element type."""
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def make_head(w, max_B: int = 64, max_K: int | None = None, projection: str = "auto"):
    from centroid_masked_sparse_amd import Head
    C = to_device(w.C, w.dtype)
    E = to_device(w.E, w.dtype)
    equal = np.all(np.diff(w.offsets) == w.V // w.Nc) and w.V % w.Nc == 0
    head = Head(C, E, w.tos, None if equal else w.offsets, max_B=max_B,
                max_K=max_K if max_K is not None else w.Nc,
                projection=projection if w.dtype == "bf16" else "auto")
    return head


def rows(w, B: int):
    """The first B hidden rows (repeating the 64 drawn rows if B > 64)."""
    h = w.h
    if B > h.shape[0]:
        reps = -(-B // h.shape[0])
        h = np.concatenate([h] * reps, axis=0)
    return np.ascontiguousarray(h[:B])


def f32_bits(t) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)
