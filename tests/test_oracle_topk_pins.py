"""Pins for the oracle's full-vocabulary top-k and Hit@k ("Cut Binary Cross Entropy", Section III-E: the
evaluation projects hidden states to full-vocabulary logits, ranks the items, and counts a user as a hit when
one of the held-out items is among the top 8). Ranking: larger logit first, smaller item id among equal logits.

* Brute force: numpy materialises the dense logits and sorts every row (lexicographic on (-z, id)).
* Closed forms: E[v] = v e_1 and H[r] = a_r e_1 give z = a_r v, so the top k are the last k ids (a_r > 0) or
  the first k (a_r < 0); identical embeddings make every logit equal, so the first k ids win (the tie rule).
* Hits: the number of returned ids that are positives, checked against the sets; masked rows give -1 / -inf / 0.
* A planted mistake (ties broken towards the larger id) must fail a pin.
"""
import numpy as np
import torch

import oracle
from vocabulary_label_bce_amd import workloads as W


def _sets(p):
    ro = p["row_offsets"].numpy()
    ids = p["item_ids"].numpy()
    return [set(ids[ro[r]:ro[r + 1]].tolist()) for r in range(len(ro) - 1)]


def pin_brute_force(plant=0):
    bad = 0
    for dtype, seed, k in (("f32", 1, 5), ("bf16", 2, 8), ("f32", 3, 1)):
        p = W.custom_problem(12, 40, 7, dtype=dtype, seed=seed, h_std=0.8, e_std=0.8, pos_per_row=(0, 6),
                             mask_frac=0.25)
        E = p["E"].clone()
        E[11] = E[23]  # two items with identical logits in every row
        p["E"] = E
        got = oracle.topk(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], k, plant=plant)
        Z = p["H"].double().numpy() @ p["E"].double().numpy().T
        sets = _sets(p)
        for r in range(Z.shape[0]):
            if not p["row_mask"][r]:
                bad += int((got["ids"][r] != -1).any() or np.isfinite(got["vals"][r]).any() or got["hits"][r] != 0)
                continue
            order = np.lexsort((np.arange(Z.shape[1]), -Z[r]))[:k]
            bad += int((got["ids"][r] != order).any())
            bad += int(not np.allclose(got["vals"][r], Z[r, order], rtol=1e-12, atol=1e-12))
            bad += int(got["hits"][r] != len(set(order.tolist()) & sets[r]))
    return bad


def pin_ties(plant=0):
    p = W.custom_problem(5, 30, 4, dtype="f32", seed=4, pos_per_row=(1, 3))
    E = torch.ones_like(p["E"]) * 0.25
    got = oracle.topk(p["H"], E, p["row_offsets"], p["item_ids"], p["row_mask"], 6, plant=plant)
    return int((got["ids"] != np.arange(6)).sum())


def test_brute_force():
    assert pin_brute_force() == 0


def test_tie_rule():
    assert pin_ties() == 0


def test_closed_form_ramp():
    R, V, D, k = 6, 50, 3, 4
    H = torch.zeros(R, D)
    a = torch.tensor([1.0, -2.0, 0.5, -0.25, 3.0, -1.0])
    H[:, 0] = a
    E = torch.zeros(V, D)
    E[:, 0] = torch.arange(V, dtype=torch.float32)
    ro = torch.zeros(R + 1, dtype=torch.int32)
    got = oracle.topk(H, E, ro, torch.zeros(0, dtype=torch.int32), torch.ones(R, dtype=torch.uint8), k)
    for r in range(R):
        want = np.arange(V - 1, V - 1 - k, -1) if a[r] > 0 else np.arange(k)
        assert (got["ids"][r] == want).all()
        assert np.allclose(got["vals"][r], a[r].item() * want)
    assert (got["hits"] == 0).all()


def test_row_subset_and_hits_on_planted_positive():
    p = W.custom_problem(9, 60, 5, dtype="f32", seed=6, h_std=0.9, e_std=0.9, pos_per_row=(0, 0))
    full = oracle.topk(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], 3)
    # make each row's best item its only positive: every row is a hit with exactly one hit
    best = full["ids"][:, 0]
    ro = torch.arange(10, dtype=torch.int32)
    ids = torch.from_numpy(best.astype(np.int32))
    got = oracle.topk(p["H"], p["E"], ro, ids, p["row_mask"], 3)
    assert (got["hits"] == 1).all()
    sub = oracle.topk(p["H"], p["E"], ro, ids, p["row_mask"], 3, rows=[7, 2])
    assert (sub["ids"] == got["ids"][[7, 2]]).all() and (sub["hits"] == 1).all()


def test_planted_tie_break_is_caught():
    """9: ties broken towards the larger item id."""
    assert pin_brute_force(plant=9) > 0 or pin_ties(plant=9) > 0
