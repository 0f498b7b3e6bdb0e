"""Dense padded targets -> CSR: the oracle's definition against a hand-worked fixture and invariants (CPU);
the library's cutbce_targets_to_csr against that definition, bit for bit, and the Listing-1 call shape
end to end (GPU)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "targets_to_csr_example.json")


def test_oracle_matches_hand_worked_example():
    g = json.load(open(GOLDEN))
    ro, ids = oracle.targets_to_csr(np.array(g["targets"]), g["pad_id"])
    assert ro.tolist() == g["row_offsets"]
    assert ids.tolist() == g["item_ids"]


def test_oracle_invariants():
    rng = np.random.default_rng(3)
    t = rng.integers(-1, 50, size=(6, 5, 7))
    t[2, 3] = -1  # an all-padding row
    ro, ids = oracle.targets_to_csr(t, -1)
    flat = t.reshape(-1, 7)
    assert ro[0] == 0 and ro[-1] == ids.size == int((flat != -1).sum())
    assert (np.diff(ro) == (flat != -1).sum(1)).all()
    for r in range(flat.shape[0]):
        assert ids[ro[r]:ro[r + 1]].tolist() == [x for x in flat[r].tolist() if x != -1]
    # another pad value
    ro2, ids2 = oracle.targets_to_csr(t, 7)
    assert ro2[-1] == int((flat != 7).sum())


@pytest.mark.gpu
@pytest.mark.parametrize("shape,pad,frac", [((4, 16, 8), -1, 0.3), ((3, 5, 1), 0, 0.5), ((7, 33, 13), 11, 0.9),
                                            ((2, 3, 0), -1, 0.0), ((128, 200, 8), -1, 0.2)])
def test_device_conversion_is_exact(shape, pad, frac):
    from vocabulary_label_bce_amd.ops import dense_to_csr

    rng = np.random.default_rng(sum(shape))
    t = rng.integers(0, 1000, size=shape).astype(np.int32)
    if t.size:
        t[rng.random(shape) < frac] = pad
        t.reshape(-1, shape[-1])[1] = pad  # an all-padding row
    ro_ref, ids_ref = oracle.targets_to_csr(t, pad)
    ro, ids = dense_to_csr(torch.from_numpy(t).cuda(), pad)
    torch.cuda.synchronize()
    ro = ro.cpu().numpy()
    assert ro.tolist() == ro_ref.tolist()
    assert ids.cpu().numpy()[: ro[-1]].tolist() == ids_ref.tolist()


@pytest.mark.gpu
def test_listing1_call_shape_matches_oracle():
    from vocabulary_label_bce_amd.ops import cut_binary_cross_entropy

    rng = np.random.default_rng(9)
    Bn, N, L, D, V = 3, 40, 6, 64, 1500
    A = torch.from_numpy(rng.standard_normal((Bn, N, D)).astype(np.float32) * 0.3).to(torch.bfloat16)
    E = torch.from_numpy(rng.standard_normal((V, D)).astype(np.float32) * 0.3).to(torch.bfloat16)
    t = rng.integers(0, V, size=(Bn, N, L)).astype(np.int32)
    t[rng.random(t.shape) < 0.4] = -1
    w = (rng.random((Bn, N)) > 0.2).astype(np.float32)
    Ad = A.cuda().requires_grad_(True)
    Ed = E.cuda().requires_grad_(True)
    loss = cut_binary_cross_entropy(Ad, Ed, torch.from_numpy(t).cuda(), torch.from_numpy(w).cuda())
    loss.backward()
    torch.cuda.synchronize()
    ro, ids = oracle.targets_to_csr(t, -1)
    ref = oracle.full(A.reshape(-1, D), E, ro, ids, (w.reshape(-1) != 0).astype(np.uint8))
    assert abs(loss.item() - ref["loss"]) <= 1e-4 * abs(ref["loss"])
    dH = Ad.grad.double().cpu().numpy().reshape(-1, D)
    assert np.abs(dH - ref["dH"]).max() <= 2e-2 * np.abs(ref["dH"]).max()
    dE = Ed.grad.double().cpu().numpy()
    assert np.abs(dE - ref["dE"]).max() <= 2e-2 * np.abs(ref["dE"]).max()


@pytest.mark.gpu
def test_capacity_sized_ids_are_ignored_past_the_last_offset():
    from vocabulary_label_bce_amd import binding as B
    from vocabulary_label_bce_amd import workloads as W
    from vocabulary_label_bce_amd.ops import Workspace

    p = {k: v.cuda() for k, v in W.custom_problem(90, 700, 64, dtype="bf16", seed=41, h_std=0.4, e_std=0.4,
                                                   pos_per_row=(1, 6), mask_frac=0.1).items()}
    nnz = p["item_ids"].numel()
    padded = torch.full((nnz + 37,), 123456, dtype=torch.int32, device="cuda")  # out-of-range garbage past nnz
    padded[:nnz] = p["item_ids"]
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.validate_targets(B.problem_of(p["H"], p["E"], padded), p["row_offsets"], padded, bad)
    outs = []
    for ids in (p["item_ids"], padded):
        w = Workspace(p["H"], p["E"], ids, want_row_loss=True)
        w.forward(p["H"], p["E"], p["row_offsets"], ids, p["row_mask"])
        dH, dE = w.backward(p["H"], p["E"], p["row_offsets"], ids, p["row_mask"])
        outs.append((w.loss.clone(), dH.clone(), dE.clone()))
    torch.cuda.synchronize()
    assert bad.item() == 0
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
