"""Writes fullsize_losses.json: the float64 oracle's loss over every valid row of the full-size workloads.

    python tests/golden/make_fullsize_losses.py

Inputs come from the seeded generators in their host-independent form (workloads.make_problem(...,
portable=True): NumPy PCG64 draws), so the GPU tests regenerate the very same values on any machine; the values
come from the oracle alone (oracle.full without gradients). A checksum of the inputs is stored with each loss
so that a test notices if the generators ever change. The losses take minutes
of CPU time (every (row, item) logit of V = 876,000 items), which is why they are stored instead of being
recomputed by each GPU test run.
"""
from __future__ import annotations

import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from vocabulary_label_bce_amd import workloads as W  # noqa: E402

CONFIGS = ["v100k", "posdense", "sasrec876k"]


def checksum(p) -> dict:
    """Float64 sums of the inputs (the values the oracle sees) and the target sizes."""
    H = p["H"].float().double()
    E = p["E"].float().double()
    return dict(H_sum=float(H.sum()), H_abs_sum=float(H.abs().sum()), E_sum=float(E.sum()),
                E_abs_sum=float(E.abs().sum()), nnz=int(p["item_ids"].numel()),
                ids_sum=int(p["item_ids"].long().sum()), valid_rows=int(p["row_mask"].long().sum()))


def main():
    out = {"source": "oracle.full(grads=False) over workloads.make_problem(name, device='cpu', portable=True)",
           "configs": {}}
    for name in CONFIGS:
        t0 = time.time()
        p = W.make_problem(name, device="cpu", portable=True)
        ref = oracle.full(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], grads=False)
        out["configs"][name] = dict(checksum=checksum(p), loss=ref["loss"], excess=ref["loss"] - math.log(2.0),
                                    row_loss_sum=float(np.sum(ref["row_loss"])),
                                    oracle_seconds=round(time.time() - t0, 1), threads=oracle.num_threads())
        print(name, out["configs"][name], flush=True)
    with open(os.path.join(HERE, "fullsize_losses.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
