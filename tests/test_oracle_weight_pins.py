"""Pins for the oracle's weighted rows (the per-position `weights` of the paper's API call, Listing 1 of "Cut
Binary Cross Entropy", read as a weight per row that turns the average over positions after Eq. (4) into a
weighted average: s = 1 / (W V) with W the summed weight of the valid rows).

Each check ties the weighted path to something other than itself:

* integer weights are row repetition: a row of weight k counts as k copies of an unweighted row (unweighted
  path of the oracle, itself pinned in test_oracle_pins), so loss and dE must match and dH[r] must be k times
  the dH of one copy;
* closed forms at E = 0 and H = 0 (every logit 0): loss ln 2 for any weights; the gradients reduce to the
  weighted rank-1 background (1/2) and the weighted target corrections;
* fifth-order finite differences of the weighted loss, on inputs where every perturbation is exact;
* invariants: scaling all weights leaves every output unchanged; 0/1 weights equal the mask; unit weights
  equal no weights, bit for bit.
* Planted mistakes: the normaliser ignoring the weights (plant 6) and dE ignoring them (plant 7) must each
  fail a pin.
"""
import math

import numpy as np
import pytest

import oracle
from vocabulary_label_bce_amd import workloads as W


def _problem(R=9, V=37, D=5, seed=31, mask_frac=0.25):
    return W.custom_problem(R, V, D, dtype="f32", seed=seed, h_std=0.7, e_std=0.9, pos_per_row=(0, 5),
                            mask_frac=mask_frac, dup_frac=0.3)


def _csr(p):
    ro = p["row_offsets"].numpy()
    ids = p["item_ids"].numpy()
    return [ids[ro[r]:ro[r + 1]] for r in range(len(ro) - 1)]


def _sets(p):
    return [set(x.tolist()) for x in _csr(p)]


def pin_w_duplicate_rows(plant=0):
    """Integer weights 0..3 against the problem in which each valid row appears weight-many times."""
    p = _problem()
    R = p["H"].shape[0]
    m = p["row_mask"].numpy()
    rng = np.random.default_rng(5)
    w = rng.integers(0, 4, R).astype(np.float64)
    w[np.flatnonzero(m)[:2]] = [0.0, 3.0]  # a valid row of weight 0 and one of weight 3
    a = oracle.full(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], g=1.3, plant=plant,
                    row_weight=w)
    lists = _csr(p)
    H = p["H"].numpy()
    copies, rows_h, rows_ids = {}, [], []
    for r in range(R):
        if m[r]:
            for _ in range(int(w[r])):
                copies.setdefault(r, len(rows_h))
                rows_h.append(H[r])
                rows_ids.append(lists[r])
    ro2 = np.concatenate([[0], np.cumsum([len(x) for x in rows_ids])]).astype(np.int32)
    ids2 = np.concatenate(rows_ids).astype(np.int32)
    H2 = np.stack(rows_h).astype(np.float32)
    b = oracle.full(H2, p["E"], ro2, ids2, np.ones(len(rows_h), np.uint8), g=1.3, plant=plant)
    dH_ref = np.zeros_like(a["dH"])
    for r, k in copies.items():
        dH_ref[r] = w[r] * b["dH"][k]
    return max(abs(a["loss"] - b["loss"]) / abs(b["loss"]),
               np.abs(a["dE"] - b["dE"]).max() / np.abs(b["dE"]).max(),
               np.abs(a["dH"] - dH_ref).max() / np.abs(dH_ref).max())


def _real_weights(R, seed):
    return np.random.default_rng(seed).uniform(0.2, 3.0, R)


def pin_w_zero_E(plant=0, g=1.7):
    p = _problem(seed=32)
    H = p["H"].numpy().astype(np.float64)
    E0 = np.zeros_like(p["E"].numpy())
    m = p["row_mask"].numpy()
    R, V = H.shape[0], E0.shape[0]
    w = _real_weights(R, 6)
    out = oracle.full(p["H"], E0, p["row_offsets"], p["item_ids"], p["row_mask"], g=g, plant=plant, row_weight=w)
    wv = np.where(m == 1, w, 0.0)
    s = 1.0 / (wv.sum() * V)
    sets = _sets(p)
    half = 0.5 * (wv[:, None] * H).sum(0)
    dE_ref = np.zeros((V, H.shape[1]))
    for v in range(V):
        corr = sum((wv[r] * H[r] for r in range(R) if m[r] and v in sets[r]), np.zeros(H.shape[1]))
        dE_ref[v] = g * s * (half - corr)
    return max(abs(out["loss"] - math.log(2.0)) / math.log(2.0),
               np.abs(out["dH"]).max(),
               np.abs(out["dE"] - dE_ref).max() / np.abs(dE_ref).max())


def pin_w_zero_H(plant=0, g=-0.6):
    p = _problem(seed=33)
    E = p["E"].numpy().astype(np.float64)
    H0 = np.zeros_like(p["H"].numpy())
    m = p["row_mask"].numpy()
    R, V = H0.shape[0], E.shape[0]
    w = _real_weights(R, 7)
    out = oracle.full(H0, p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], g=g, plant=plant, row_weight=w)
    wv = np.where(m == 1, w, 0.0)
    s = 1.0 / (wv.sum() * V)
    sets = _sets(p)
    dH_ref = np.zeros((R, E.shape[1]))
    for r in range(R):
        if m[r]:
            dH_ref[r] = g * s * wv[r] * (0.5 * E.sum(0) - sum((E[v] for v in sets[r]), np.zeros(E.shape[1])))
    return max(abs(out["loss"] - math.log(2.0)) / math.log(2.0),
               np.abs(out["dE"]).max(),
               np.abs(out["dH"] - dH_ref).max() / np.abs(dH_ref).max())


def pin_w_finite_differences(plant=0):
    """5-point central differences of the weighted oracle loss vs its dH and dE (g = 1)."""
    rng = np.random.default_rng(12)
    R, V, D = 4, 6, 3
    q = 2.0 ** -10  # every value and every perturbation is a multiple of 2^-10: exact in float32
    H = (np.round(rng.normal(0, 1.0, (R, D)) / q) * q).astype(np.float32)
    E = (np.round(rng.normal(0, 1.0, (V, D)) / q) * q).astype(np.float32)
    ro = np.array([0, 2, 2, 5, 6], np.int32)
    ids = np.array([1, 4, 0, 5, 0, 3], np.int32)
    m = np.array([1, 1, 0, 1], np.uint8)
    w = np.array([0.5, 2.25, 7.0, 1.5])
    out = oracle.full(H, E, ro, ids, m, plant=plant, row_weight=w)

    def L(Hx, Ex):
        return oracle.full(Hx, Ex, ro, ids, m, grads=False, plant=plant, row_weight=w)["loss"]

    eps = 8 * q
    worst = 0.0
    for which, X, G in (("H", H, out["dH"]), ("E", E, out["dE"])):
        for idx in np.ndindex(X.shape):
            vals = []
            for k in (-2, -1, 1, 2):
                Y = X.copy()
                Y[idx] += k * eps
                vals.append(L(Y, E) if which == "H" else L(H, Y))
            fd = (vals[0] - 8 * vals[1] + 8 * vals[2] - vals[3]) / (12 * eps)
            worst = max(worst, abs(fd - G[idx]) / np.abs(G).max())
    return worst


PINS = [pin_w_duplicate_rows, pin_w_zero_E, pin_w_zero_H, pin_w_finite_differences]
TOL = {pin_w_duplicate_rows: 1e-13, pin_w_zero_E: 1e-13, pin_w_zero_H: 1e-13, pin_w_finite_differences: 1e-7}


@pytest.mark.parametrize("pin", PINS, ids=[f.__name__ for f in PINS])
def test_weight_pin(pin):
    assert pin() < TOL[pin]


def test_weights_scale_free_mask_and_unit():
    p = _problem(seed=34)
    R = p["H"].shape[0]
    m = p["row_mask"].numpy()
    args = (p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"])
    w = _real_weights(R, 8)
    a = oracle.full(*args, g=0.9, row_weight=w)
    b = oracle.full(*args, g=0.9, row_weight=4.0 * w)  # a power of two: every product stays exact
    assert a["loss"] == b["loss"]
    np.testing.assert_array_equal(a["dH"], b["dH"])
    np.testing.assert_array_equal(a["dE"], b["dE"])
    np.testing.assert_array_equal(a["row_loss"], b["row_loss"])
    # 0/1 weights on an all-valid mask equal the 0/1 mask
    ones = np.ones(R, np.uint8)
    c = oracle.full(p["H"], p["E"], p["row_offsets"], p["item_ids"], ones, row_weight=m.astype(np.float64))
    d = oracle.full(*args)
    assert c["loss"] == d["loss"]
    np.testing.assert_array_equal(c["dH"], d["dH"])
    np.testing.assert_array_equal(c["dE"], d["dE"])
    # unit weights equal no weights
    e = oracle.full(*args, row_weight=np.ones(R))
    assert e["loss"] == d["loss"]
    np.testing.assert_array_equal(e["dH"], d["dH"])
    np.testing.assert_array_equal(e["dE"], d["dE"])
    # every valid row of weight 0: zero loss and gradients
    z = oracle.full(*args, row_weight=np.zeros(R))
    assert z["loss"] == 0.0 and not z["dH"].any() and not z["dE"].any()


def test_weighted_subset_entry_points_agree_with_full():
    p = _problem(seed=35)
    R = p["H"].shape[0]
    w = _real_weights(R, 9)
    args = (p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"])
    a = oracle.full(*args, g=0.75, row_weight=w)
    rr = [0, 3, 5, 8]
    b = oracle.rows(*args, rr, g=0.75, row_weight=w)
    c = oracle.items(*args, [1, 7, 12], g=0.75, row_weight=w)
    np.testing.assert_array_equal(b["row_loss"], a["row_loss"][rr])
    np.testing.assert_array_equal(b["dH"], a["dH"][rr])
    np.testing.assert_array_equal(c["dE"], a["dE"][[1, 7, 12]])


@pytest.mark.parametrize("plant", [6, 7])
def test_planted_weight_mistakes_are_caught(plant):
    """6: the normaliser ignores the weights; 7: dE ignores the weights."""
    caught = [f.__name__ for f in PINS if not f(plant=plant) < TOL[f]]
    assert caught, f"planted mistake {plant} passed every weight pin"
