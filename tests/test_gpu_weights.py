"""Weighted rows on the GPU (row_weight of cutbce_forward / cutbce_backward, and the per-position weights of
the Listing-1 call shape) against the float64 oracle's weighted average. Tolerances as in test_gpu_parity.
The slot-packed H operand of the dE sweep carries w_r H[r] rounded once to the element type, which stays
inside the bf16 gradient tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle
from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace, cut_binary_cross_entropy, cut_bce

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: dict(loss=1e-4, grad=2e-2, excess=1e-2, row=1e-4),
       torch.float32: dict(loss=1e-5, grad=1e-4, excess=1e-4, row=1e-5)}


def _weights(R, seed, zero_frac=0.15):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.1, 3.0, R).astype(np.float32)
    w[rng.random(R) < zero_frac] = 0.0
    return w


def _run(p, w, g=1.0, use_saved=True):
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    wt = None if w is None else torch.from_numpy(w).cuda()
    ws = Workspace(d["H"], d["E"], d["item_ids"], want_row_loss=True, save_dh=True)
    ws.forward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"], row_weight=wt)
    gt = torch.tensor([g], dtype=torch.float32, device="cuda")
    dH, dE = ws.backward(d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"], grad=gt,
                         use_saved=use_saved, row_weight=wt)
    torch.cuda.synchronize()
    return dict(loss=ws.loss.item(), row_loss=ws.row_loss.double().cpu().numpy(),
                dH=dH.double().cpu().numpy(), dE=dE.double().cpu().numpy())


def _check(p, got, ref):
    tol = TOL[p["H"].dtype]
    assert math.isfinite(got["loss"])
    assert abs(got["loss"] - ref["loss"]) <= tol["loss"] * abs(ref["loss"]), (got["loss"], ref["loss"])
    ex_ref = ref["loss"] - math.log(2.0)
    if abs(ex_ref) > 1e-6:
        assert abs((got["loss"] - math.log(2.0)) - ex_ref) <= tol["excess"] * abs(ex_ref)
    assert np.abs(got["row_loss"] - ref["row_loss"]).max() <= tol["row"] * max(np.abs(ref["row_loss"]).max(), 1e-30)
    for k in ("dH", "dE"):
        scale = np.abs(ref[k]).max()
        err = np.abs(got[k] - ref[k]).max()
        assert err <= tol["grad"] * scale, f"{k}: err {err:.3e} vs {tol['grad']} x {scale:.3e}"


CASES = [
    ("bf16_d128", dict(R=300, V=5001, D=128, dtype="bf16", seed=61, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                       mask_frac=0.2, dup_frac=0.2), 0.5),
    ("f32_d64", dict(R=200, V=3001, D=64, dtype="f32", seed=62, h_std=0.5, e_std=0.5, pos_per_row=(0, 6),
                     mask_frac=0.1), -1.25),
    ("bf16_d512", dict(R=150, V=555, D=512, dtype="bf16", seed=63, h_std=0.1, e_std=0.2, pos_per_row=(1, 30),
                       mask_frac=0.1), 1.0),
    ("f32_d256", dict(R=100, V=600, D=256, dtype="f32", seed=64, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                      mask_frac=0.1), 2.0),
    ("f32_paper_normal", dict(R=96, V=1500, D=64, dtype="f32", seed=65, h_std=1.0, e_std=1.0, pos_per_row=(8, 8),
                              mask_frac=0.1), 1.0),
]


@pytest.mark.parametrize("name,kw,g", CASES, ids=[c[0] for c in CASES])
def test_weighted_rows_match_oracle(name, kw, g):
    p = W.custom_problem(**kw)
    w = _weights(kw["R"], kw["seed"])
    ref = oracle.full(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], g=g, row_weight=w)
    _check(p, _run(p, w, g=g), ref)


def test_weighted_recompute_path_matches_saved():
    p = W.custom_problem(250, 2500, 128, dtype="bf16", seed=66, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                         mask_frac=0.2)
    w = _weights(250, 66)
    a = _run(p, w, g=0.5)
    b = _run(p, w, g=0.5, use_saved=False)
    np.testing.assert_array_equal(a["dH"], b["dH"])
    np.testing.assert_array_equal(a["dE"], b["dE"])


def test_unit_weights_are_bitwise_no_weights_and_binary_weights_the_mask():
    p = W.custom_problem(270, 3000, 64, dtype="bf16", seed=67, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                         mask_frac=0.25)
    R = 270
    a = _run(p, None, g=0.7)
    b = _run(p, np.ones(R, np.float32), g=0.7)
    assert a["loss"] == b["loss"]
    for k in ("row_loss", "dH", "dE"):
        np.testing.assert_array_equal(a[k], b[k])
    # the mask as 0/1 weights over an all-valid mask: same mathematics, other row grouping in the sweeps
    q = dict(p)
    q["row_mask"] = torch.ones_like(p["row_mask"])
    c = _run(q, p["row_mask"].numpy().astype(np.float32), g=0.7)
    assert abs(c["loss"] - a["loss"]) <= 1e-6 * abs(a["loss"])
    m = p["row_mask"].numpy() == 1
    for k in ("dH", "dE"):
        assert np.abs(c[k] - a[k]).max() <= 1e-3 * np.abs(a[k]).max()
    assert not c["dH"][~m].any()


def test_all_weights_zero():
    p = W.custom_problem(64, 700, 64, dtype="f32", seed=68, h_std=0.5, e_std=0.5, pos_per_row=(1, 4))
    got = _run(p, np.zeros(64, np.float32))
    assert got["loss"] == 0.0 and not got["dH"].any() and not got["dE"].any()


def test_autograd_and_listing1_weights_match_oracle():
    rng = np.random.default_rng(69)
    Bn, N, L, D, V = 3, 40, 6, 64, 1500
    A = torch.from_numpy(rng.standard_normal((Bn, N, D)).astype(np.float32) * 0.3).to(torch.bfloat16)
    E = torch.from_numpy(rng.standard_normal((V, D)).astype(np.float32) * 0.3).to(torch.bfloat16)
    t = rng.integers(0, V, size=(Bn, N, L)).astype(np.int32)
    t[rng.random(t.shape) < 0.4] = -1
    w = rng.uniform(0.25, 2.0, (Bn, N)).astype(np.float32)
    w[rng.random((Bn, N)) < 0.2] = 0.0
    Ad = A.cuda().requires_grad_(True)
    Ed = E.cuda().requires_grad_(True)
    loss = cut_binary_cross_entropy(Ad, Ed, torch.from_numpy(t).cuda(), torch.from_numpy(w).cuda())
    (1.5 * loss).backward()
    torch.cuda.synchronize()
    ro, ids = oracle.targets_to_csr(t, -1)
    wf = w.reshape(-1)
    ref = oracle.full(A.reshape(-1, D), E, ro, ids, (wf != 0).astype(np.uint8), g=1.5, row_weight=wf)
    assert abs(loss.item() - ref["loss"]) <= 1e-4 * abs(ref["loss"])
    dH = Ad.grad.double().cpu().numpy().reshape(-1, D)
    assert np.abs(dH - ref["dH"]).max() <= 2e-2 * np.abs(ref["dH"]).max()
    dE = Ed.grad.double().cpu().numpy()
    assert np.abs(dE - ref["dE"]).max() <= 2e-2 * np.abs(ref["dE"]).max()
    # cut_bce with explicit row weights gives the same loss
    H2 = A.reshape(-1, D).cuda()
    l2 = cut_bce(H2, E.cuda(), torch.from_numpy(ro).cuda(), torch.from_numpy(ids).cuda(),
                 torch.from_numpy((wf != 0).astype(np.uint8)).cuda(), row_weight=torch.from_numpy(wf).cuda())
    assert abs(l2.item() - ref["loss"]) <= 1e-4 * abs(ref["loss"])


def test_cut_metrics_ignore_weights():
    p = {k: v.cuda() for k, v in W.custom_problem(180, 2000, 64, dtype="bf16", seed=70, h_std=0.5, e_std=0.5,
                                                    pos_per_row=(1, 8), mask_frac=0.2).items()}
    out = []
    for wt in (None, torch.from_numpy(_weights(180, 70)).cuda()):
        ws = Workspace(p["H"], p["E"], p["item_ids"], want_metrics=True)
        ws.forward(p["H"], p["E"], p["row_offsets"], p["item_ids"], p["row_mask"], row_weight=wt)
        torch.cuda.synchronize()
        out.append(ws.metrics.cpu().clone())
    assert torch.equal(out[0], out[1])


def test_graph_replay_reads_new_weights():
    """A captured forward + backward reads the weights anew on every replay."""
    p = W.custom_problem(200, 3000, 128, dtype="bf16", seed=71, h_std=0.3, e_std=0.3, pos_per_row=(1, 6),
                         mask_frac=0.2)
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}
    args = (d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
    w1 = torch.from_numpy(_weights(200, 71)).cuda()
    w2 = torch.from_numpy(_weights(200, 72)).cuda()
    wbuf = w1.clone()
    ws = Workspace(d["H"], d["E"], d["item_ids"])
    g = torch.tensor([0.5], device="cuda")

    def step():
        ws.forward(*args, row_weight=wbuf)
        return ws.backward(*args, grad=g, row_weight=wbuf)

    refs = []
    for w in (w1, w2):
        wbuf.copy_(w)
        dH, dE = step()
        torch.cuda.synchronize()
        refs.append((ws.loss.clone(), dH.clone(), dE.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdH, gdE = step()
    torch.cuda.synchronize()
    for k in (0, 1, 0):
        wbuf.copy_((w1, w2)[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ws.loss, refs[k][0])
        assert torch.equal(gdH, refs[k][1])
        assert torch.equal(gdE, refs[k][2])
