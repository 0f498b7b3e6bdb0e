"""The first launch of each sweep in a process (cold instruction and address-translation caches, waves far out of
step) must give the same bits as every later launch. Each unit of the interleaved engine reads step 0's ring
slot before its first loop iteration, and that slot is refilled in iteration 1: a barrier separates the two, and
without it a wave that ran ahead overwrote the block under a slower one (seen only on first launches). This file
is named to run before the other GPU tests, so that its first calls are the process's first sweep launches."""
import pytest
import torch

from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [128, 64])
def test_first_launch_matches_later_launches(D):
    p = W.custom_problem(700, 20000, D, dtype="bf16", seed=81, h_std=0.3, e_std=0.3, pos_per_row=(1, 10),
                         mask_frac=0.15, dup_frac=0.2)
    d = {k: v.cuda() for k, v in p.items()}
    w = Workspace(d["H"], d["E"], d["item_ids"], want_row_loss=True, save_dh=True)
    args = (d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
    g = torch.tensor([0.5], device="cuda")
    runs = []
    for _ in range(4):
        w.forward(*args)
        dH, dE = w.backward(*args, grad=g, reuse=True)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (w.loss, w.row_loss, w.dh_saved, dH, dE)])
    for later in runs[1:]:
        for name, a, b in zip(("loss", "row_loss", "dh_saved", "dH", "dE"), runs[0], later):
            assert torch.equal(a, b), name
