"""The 16-owner forward's persistent unit loop (bf16, D = 256 and 512). With 256 resident workgroups the workload
shapes give each workgroup at most one (vocabulary split, row tile) unit; these shapes have about 300 row tiles,
so the device picks 3 vocabulary splits and each workgroup runs three or four units in a row, reusing its rings,
accumulators and (for the paired D = 512 waves) the partial-logit exchange slots. Sampled rows and items against
the float64 oracle, as in test_gpu_fullsize, and the same bits with Cut Metrics (the one-wave D = 512 kernel) as
without."""
import numpy as np
import pytest
import torch

import test_gpu_fullsize as F
from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,R", [(512, 20480), (256, 40960)])
def test_many_units_per_workgroup(D, R):
    p = W.custom_problem(R, 1024, D, dtype="bf16", seed=91 + D, h_std=1.0 / np.sqrt(D), e_std=0.05,
                         pos_per_row=(1, 6), mask_frac=0.05)
    rows, items = F._samples(p, 128, 256, seed=5)
    got = F._run_gpu(p, rows, items)
    m = p["row_mask"].numpy()
    assert got["loss"] == pytest.approx(got["row_loss"][m == 1].sum() / (m.sum() * p["E"].shape[0]), rel=1e-5)
    F._sampled_check(p, rows, items, got)

    d = {k: p[k].cuda() for k in ("H", "E", "row_offsets", "item_ids", "row_mask")}
    outs = []
    for met in (False, True):
        w = Workspace(d["H"], d["E"], d["item_ids"], want_row_loss=True, save_dh=True, want_metrics=met)
        w.forward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
        torch.cuda.synchronize()
        outs.append((w.loss.clone(), w.row_loss.clone(), w.dh_saved.clone()))
        del w
    assert all(torch.equal(a, b) for a, b in zip(*outs))
