"""GPU Cut Metrics ("Cut Binary Cross Entropy", Section III-D): TP, FP, FN, TN per row from the forward sweep,
through the C ABI, against the float64 oracle.

The prediction is z > 0. The GPU evaluates z in float32 from the same inputs, so its sign may differ from the
float64 sign only where |z| is within the float32 dot-product error bound eps = (D + 2) 2^-24 |H_r| |E_v|
(Cauchy-Schwarz bound on sum_d |h_d e_d|, doubled); the oracle counts those items per row, and every count
must match to within that number. Integer identities hold exactly: TP + FN = |P_r| (distinct ids) and
TP + FP + FN + TN = V; masked rows are all zero. Turning metrics on changes no other output bit.
"""
import numpy as np
import pytest
import torch

import oracle
from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace

pytestmark = pytest.mark.gpu


def _eps(p):
    H = p["H"].double()
    E = p["E"].double()
    D = H.shape[1]
    return 2.0 * (D + 2) * 2.0 ** -24 * float(H.norm(dim=1).max()) * float(E.norm(dim=1).max())


def _forward(p, metrics=True):
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    w = Workspace(d["H"], d["E"], d["item_ids"], want_row_loss=True, save_dh=True, want_metrics=metrics)
    w.forward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
    torch.cuda.synchronize()
    return w


def _distinct(p):
    ro = p["row_offsets"].numpy()
    ids = p["item_ids"].numpy()
    V = p["E"].shape[0]
    return np.array([len({x for x in ids[ro[r]:ro[r + 1]].tolist() if 0 <= x < V}) for r in range(len(ro) - 1)])


def _check(p, got, ref, rows):
    V = p["E"].shape[0]
    m = p["row_mask"].numpy()[rows]
    npos = _distinct(p)[rows]
    assert (got[m == 0] == 0).all()
    g, r = got[m == 1], ref[m == 1]
    assert (g.sum(1) == V).all()
    assert (g[:, 0] + g[:, 2] == npos[m == 1]).all()
    assert (np.abs(g - r[:, :4]) <= r[:, 4:5]).all(), np.abs(g - r[:, :4]).max()


CASES = [
    ("bf16_d64_ragged", dict(R=300, V=1000, D=64, dtype="bf16", seed=21, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                             mask_frac=0.2, dup_frac=0.2)),
    ("bf16_d128_unaligned", dict(R=63, V=4097, D=128, dtype="bf16", seed=22, h_std=0.3, e_std=0.3,
                                 pos_per_row=(0, 6), mask_frac=0.1, dup_frac=0.3)),
    ("bf16_d256", dict(R=200, V=777, D=256, dtype="bf16", seed=23, h_std=0.2, e_std=0.2, pos_per_row=(1, 8),
                       mask_frac=0.1)),
    ("bf16_d512", dict(R=150, V=555, D=512, dtype="bf16", seed=24, h_std=0.1, e_std=0.2, pos_per_row=(1, 30),
                       mask_frac=0.05)),
    ("f32_d64", dict(R=257, V=513, D=64, dtype="f32", seed=25, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                     mask_frac=0.1, dup_frac=0.2)),
    ("f32_d128", dict(R=200, V=700, D=128, dtype="f32", seed=26, h_std=0.3, e_std=0.3, pos_per_row=(1, 8))),
    ("bf16_paper_normal", dict(R=128, V=2048, D=128, dtype="bf16", seed=27, h_std=1.0, e_std=1.0,
                               pos_per_row=(8, 8), mask_frac=0.1)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_metrics_match_oracle(name, kw):
    p = W.custom_problem(**kw)
    E = p["E"].clone()
    E[5] = 0  # an item whose logits are exactly 0 (predicted negative on both sides)
    E[kw["V"] - 1] = 0
    p["E"] = E
    w = _forward(p)
    got = w.metrics.cpu().numpy().astype(np.int64)
    ref = oracle.metrics(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], eps=_eps(p))
    _check(p, got, ref, np.arange(kw["R"]))


@pytest.mark.parametrize("D", [128, 256, 512])
def test_metrics_leave_other_outputs_unchanged(D):
    # at D = 512 the two calls run different forward kernels (one wave per SIMD with Cut Metrics, paired waves
    # without), which must still agree bit for bit
    p = W.custom_problem(300, 3000, D, dtype="bf16", seed=31, h_std=0.4, e_std=0.4, pos_per_row=(1, 8),
                         mask_frac=0.2, dup_frac=0.2)
    a = _forward(p, metrics=True)
    b = _forward(p, metrics=False)
    assert a.loss.item() == b.loss.item()
    assert torch.equal(a.row_loss, b.row_loss)
    assert torch.equal(a.dh_saved, b.dh_saved)


def test_metrics_all_masked_and_zero_embeddings():
    p = W.custom_problem(70, 900, 64, dtype="bf16", seed=32, h_std=0.4, e_std=0.4, pos_per_row=(1, 5))
    p["row_mask"] = torch.zeros_like(p["row_mask"])
    w = _forward(p)
    assert (w.metrics.cpu() == 0).all()
    p = W.custom_problem(70, 900, 64, dtype="bf16", seed=33, h_std=0.4, e_std=0.4, pos_per_row=(1, 5),
                         mask_frac=0.3)
    p["E"] = torch.zeros_like(p["E"])  # every logit is 0: nothing is predicted positive
    w = _forward(p)
    got = w.metrics.cpu().numpy()
    m = p["row_mask"].numpy()
    npos = _distinct(p)
    assert (got[m == 1, 0] == 0).all() and (got[m == 1, 1] == 0).all()
    assert (got[m == 1, 2] == npos[m == 1]).all() and (got[m == 1, 3] == 900 - npos[m == 1]).all()


def test_metrics_sasrec876k_sampled():
    cfg = W.CONFIGS["sasrec876k"]
    p = W.make_problem(cfg, device="cuda")
    w = Workspace(p["H"], p["E"], p["item_ids"], want_metrics=True, save_dh=False)
    w.forward(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"])
    torch.cuda.synchronize()
    cpu = {k: v.cpu() for k, v in p.items() if torch.is_tensor(v)}
    m = cpu["row_mask"].numpy()
    rng = np.random.default_rng(7)
    rows = np.concatenate([rng.choice(np.flatnonzero(m), size=12, replace=False), np.flatnonzero(m == 0)[:2]])
    ref = oracle.metrics(cpu["H"], cpu["E"], cpu["row_offsets"], cpu["item_ids"], cpu["row_mask"], rows=rows,
                         eps=_eps(cpu))
    got = w.metrics.cpu().numpy().astype(np.int64)[rows]
    _check(cpu, got, ref, rows)
