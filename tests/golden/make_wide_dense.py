"""Write ``wide_dense.json``: the dense argmax of the wide configuration.

The wide workload (d=1024, V=262144, Nc=4096 equal clusters of 64 tokens,
bf16, seed 4) is run with K = Nc, where every centroid is selected and the
sparse head's greedy token must equal the dense lm_head's argmax (ties to the
lowest token id).  The oracle's dense logits of all 64 rows take a few
minutes on one core, so this script computes them once and stores, per row,
the best and second-best token ids and their fp32 logits (bit patterns).
It calls only ``oracle`` (and ``workloads`` for the seeded inputs).

Run from the repository root: ``python tests/golden/make_wide_dense.py``.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_workload  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "wide_dense.json")


def main() -> None:
    w = make_workload("wide")
    rows = []
    for b0 in range(0, 64, 8):
        D = oracle.dense_logits(w.h[b0:b0 + 8], w.E, w.tos, w.dtype)
        for i in range(D.shape[0]):
            order = np.argsort(-D[i].astype(np.float64), kind="stable")   # ties: lowest token first
            t1, t2 = int(order[0]), int(order[1])
            rows.append({"row": b0 + i, "best": t1, "second": t2,
                         "best_logit": f"0x{int(D[i, t1].view(np.uint32)):08x}",
                         "second_logit": f"0x{int(D[i, t2].view(np.uint32)):08x}"})
        print(f"rows {b0}..{b0 + D.shape[0] - 1} done", flush=True)
    doc = {
        "source": ("Dense argmax of the wide configuration (d=1024, V=262144, Nc=4096, bf16, "
                   "seed 4; every one of its 64 hidden rows) from oracle.dense_logits: the "
                   "canonical float64 chain rounded to fp32, ties to the lowest token id.  "
                   "With K = Nc the sparse head's top token equals 'best' (the dense "
                   "lm_head's argmax, Gemma4MTP.compute_logits in the vLLM compare view).  "
                   "Written by tests/golden/make_wide_dense.py, which calls only the oracle."),
        "workload": "wide",
        "rows": rows,
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
