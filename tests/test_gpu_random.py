"""Randomised GPU parity: 24 generated problems (fixed seed) against the full float64 oracle, mixing dtype, D,
ragged R and V, masked rows, repeated ids, rows without positives and value scales. Every sixth problem has
more item tiles than workgroups that run at once, with a remainder of at most half a round (halved tail tiles
in the dE sweep); every sixth, offset by one, has more than 64 row steps (bucket blocks refilled in the dE
sweep). Tolerances as in test_gpu_parity."""
import numpy as np
import pytest
import torch

import oracle
from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: dict(loss=1e-4, grad=2e-2, row=1e-4), torch.float32: dict(loss=1e-5, grad=1e-4, row=1e-5)}


def _cases(n=24, seed=2718):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        dtype = str(rng.choice(["bf16", "f32"]))
        D = int(rng.choice([64, 128, 256] + ([512] if dtype == "bf16" else [])))
        kind = k % 6
        if kind == 0:
            D = 128
            tail = True
            R = int(rng.integers(20, 60))
            V = None  # set from the device's CU count
        elif kind == 1:
            tail = False
            R = int(rng.integers(2100, 4200))
            V = int(rng.integers(200, 900))
        else:
            tail = False
            R = int(rng.integers(1, 400))
            V = int(rng.integers(1, 6000))
        out.append(dict(R=R, V=V, D=D, dtype=dtype, seed=int(rng.integers(1 << 30)), tail=tail,
                        h_std=float(rng.choice([0.1, 0.3, 1.0])), e_std=float(rng.choice([0.1, 0.3, 1.0])),
                        pos_per_row=(0, int(rng.integers(1, 12))), mask_frac=float(rng.choice([0.0, 0.2, 0.9])),
                        dup_frac=float(rng.choice([0.0, 0.3])), g=float(rng.choice([1.0, 0.3])),
                        extra=int(rng.integers(1, 64)), cut=int(rng.integers(0, 40))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{i}-{c['dtype']}-d{c['D']}" for i, c in enumerate(CASES)])
def test_random_problem_matches_oracle(case):
    c = dict(case)
    if c.pop("tail"):
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        tile = 256 if c["dtype"] == "bf16" else 128
        c["V"] = (cus + c["extra"]) * tile - c["cut"]
    g = c.pop("g")
    for k in ("extra", "cut"):
        c.pop(k)
    p = W.custom_problem(**c)
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    w = Workspace(d["H"], d["E"], d["item_ids"], want_row_loss=True, save_dh=True)
    w.forward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
    dH, dE = w.backward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"],
                        grad=torch.tensor([g], device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.full(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], g=g)
    tol = TOL[p["H"].dtype]
    loss = w.loss.item()
    assert abs(loss - ref["loss"]) <= tol["loss"] * abs(ref["loss"]), (loss, ref["loss"])
    rl = w.row_loss.double().cpu().numpy()
    assert np.abs(rl - ref["row_loss"]).max() <= tol["row"] * max(np.abs(ref["row_loss"]).max(), 1e-30)
    for name, got in (("dH", dH), ("dE", dE)):
        r = ref[name]
        err = np.abs(got.double().cpu().numpy() - r).max()
        assert err <= tol["grad"] * np.abs(r).max(), f"{name}: err {err:.3e} vs scale {np.abs(r).max():.3e}"
