"""Pins for the oracle's Cut Metrics ("Cut Binary Cross Entropy", Section III-D): per-row TP, FP, FN, TN over
the V items with the prediction z > 0 (z = 0 predicts negative), zeros for masked rows.

* Brute force: numpy materialises the dense logits Z = H E^T and the multi-hot targets on tiny inputs, and
  counts the four cells directly.
* Closed form: with E = 0 every logit is exactly 0, so nothing is predicted positive: TP = FP = 0,
  FN = |P_r|, TN = V - |P_r| (this fixes the tie rule).
* Invariants: the four counts add up to V and TP + FN = |P_r|; negating E swaps predicted and not predicted
  (TP <-> FN, FP <-> TN) when no logit is 0; masked rows give zeros.
* A planted mistake (z >= 0 predicts positive) must fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle
from vocabulary_label_bce_amd import workloads as W


def _problem(R=11, V=17, D=6, seed=5, dtype="f32", zero_items=(3, 9)):
    p = W.custom_problem(R, V, D, dtype=dtype, seed=seed, h_std=0.8, e_std=0.9, pos_per_row=(0, 5),
                         mask_frac=0.25, dup_frac=0.3)
    E = p["E"].clone()
    for v in zero_items:  # items whose logits are exactly 0 for every row
        E[v] = 0
    p["E"] = E
    return p


def _sets(p):
    ro = p["row_offsets"].numpy()
    ids = p["item_ids"].numpy()
    return [set(ids[ro[r]:ro[r + 1]].tolist()) for r in range(len(ro) - 1)]


def _dense_counts(p):
    H = p["H"].to(torch.float64).numpy()
    E = p["E"].to(torch.float64).numpy()
    Z = H @ E.T
    R, V = Z.shape
    Y = np.zeros((R, V), bool)
    for r, s in enumerate(_sets(p)):
        Y[r, list(s)] = True
    pred = Z > 0
    out = np.stack([(pred & Y).sum(1), (pred & ~Y).sum(1), (~pred & Y).sum(1), (~pred & ~Y).sum(1)], 1)
    out[p["row_mask"].numpy() == 0] = 0
    return out


def pin_brute_force(plant=0):
    bad = 0
    for dtype, seed in (("f32", 5), ("bf16", 6), ("f32", 7)):
        p = _problem(seed=seed, dtype=dtype)
        got = oracle.metrics(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], plant=plant)
        bad += int(np.abs(got[:, :4] - _dense_counts(p)).sum())
    return bad


def pin_zero_E(plant=0):
    p = _problem()
    E0 = torch.zeros_like(p["E"])
    got = oracle.metrics(p["H"], E0, p["row_offsets"], p["item_ids"], p["row_mask"], eps=0.0, plant=plant)
    V = E0.shape[0]
    bad = 0
    for r, s in enumerate(_sets(p)):
        want = [0, 0, len(s), V - len(s), V] if p["row_mask"][r] else [0, 0, 0, 0, 0]
        bad += int(np.abs(got[r] - np.array(want)).sum())
    return bad


def test_brute_force():
    assert pin_brute_force() == 0


def test_zero_E_predicts_nothing():
    assert pin_zero_E() == 0


def test_invariants_and_negation():
    p = _problem(zero_items=())
    V = p["E"].shape[0]
    m = p["row_mask"].numpy()
    got = oracle.metrics(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], eps=0.0)
    neg = oracle.metrics(p["H"], -p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], eps=0.0)
    sets = _sets(p)
    for r in range(len(sets)):
        if not m[r]:
            assert (got[r] == 0).all() and (neg[r] == 0).all()
            continue
        assert got[r, :4].sum() == V
        assert got[r, 0] + got[r, 2] == len(sets[r])
        assert got[r, 4] == 0  # no logit is exactly 0 here
        assert list(neg[r, :4]) == [got[r, 2], got[r, 3], got[r, 0], got[r, 1]]


def test_near_zero_count_and_row_subset():
    p = _problem()
    allr = oracle.metrics(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], eps=np.inf)
    V = p["E"].shape[0]
    m = p["row_mask"].numpy()
    assert (allr[m == 1, 4] == V).all()
    sub = oracle.metrics(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], rows=[4, 0, 7],
                         eps=np.inf)
    assert (sub == allr[[4, 0, 7]]).all()


def test_near_zero_count_at_intermediate_eps():
    """Logits fixed exactly by construction (H[r] = (1, 0), E[v] = (a_v, 0), so z = a_v, powers of two): the count
    of |z| <= eps follows the list, with eps inclusive at a logit's magnitude."""
    a = np.array([0.5, -0.25, 2.0 ** -7, -(2.0 ** -6), 2.0 ** -5, 0.0625, 0.0, -(2.0 ** -9)], np.float32)
    V = a.size
    H = torch.tensor([[1.0, 0.0], [2.0, 0.0]])
    E = torch.zeros(V, 2)
    E[:, 0] = torch.from_numpy(a)
    ro = torch.tensor([0, 2, 3], dtype=torch.int32)
    ids = torch.tensor([2, 4, 0], dtype=torch.int32)
    m = torch.ones(2, dtype=torch.uint8)
    for eps, want0 in [(0.03, 4), (2.0 ** -5, 5), (2.0 ** -8, 2), (0.3, 7)]:
        got = oracle.metrics(H, E, ro, ids, m, eps=eps)
        assert got[0, 4] == want0, (eps, got[0])
        # row 1 has logits 2 a: its count is that of row 0 at eps / 2
        assert got[1, 4] == oracle.metrics(H[:1], E, ro[:2], ids, m[:1], eps=eps / 2)[0, 4]
    # predictions: z > 0 for 0.5, 2^-7, 2^-5, 0.0625; positives of row 0 are items 2 and 4 (both predicted)
    got = oracle.metrics(H, E, ro, ids, m, eps=0.0)
    assert list(got[0, :4]) == [2, 2, 0, 4]


def test_planted_tie_rule_is_caught():
    """8: a zero logit predicted positive."""
    assert pin_brute_force(plant=8) > 0 or pin_zero_E(plant=8) > 0
