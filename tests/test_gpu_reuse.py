"""cutbce_backward_reuse: the backward that reuses the row compaction and H preparation a cutbce_forward left in
its workspace must give the bits of cutbce_backward, which recomputes them (and which the parity tests check
against the float64 oracle). Covers every kernel family (bf16 D = 64 / 128 / 256 / 512, f32), row weights and
masked rows, the dE-only and dH-only calls, the recompute path for dH, a forward given no dh_saved, the autograd
front end, and replays of a captured forward + backward."""
import numpy as np
import pytest
import torch

from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace, cut_bce

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16_d64", dict(R=333, V=4097, D=64, dtype="bf16", seed=81, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                      mask_frac=0.2, dup_frac=0.2)),
    ("bf16_d128", dict(R=600, V=9001, D=128, dtype="bf16", seed=82, h_std=1.0, e_std=0.3, pos_per_row=(0, 6),
                       mask_frac=0.3)),
    ("bf16_d256", dict(R=200, V=3000, D=256, dtype="bf16", seed=83, h_std=0.2, e_std=0.2, pos_per_row=(1, 4))),
    ("bf16_d512", dict(R=150, V=1555, D=512, dtype="bf16", seed=84, h_std=0.1, e_std=0.2, pos_per_row=(1, 40),
                       mask_frac=0.05)),
    ("f32_d64", dict(R=257, V=3001, D=64, dtype="f32", seed=85, h_std=0.5, e_std=0.5, pos_per_row=(0, 6),
                     mask_frac=0.1)),
    ("f32_d256", dict(R=120, V=1000, D=256, dtype="f32", seed=86, h_std=0.2, e_std=0.2, pos_per_row=(1, 5))),
]


def _dev(p):
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in p.items()}


def _weights(R, seed):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.1, 3.0, R).astype(np.float32)
    w[rng.random(R) < 0.15] = 0.0
    return torch.from_numpy(w).cuda()


def _step(w, d, g, wt, reuse, use_saved=True, want_dH=True, want_dE=True):
    args = (d["H"], d["E"], d["row_offsets"], d["item_ids"], d["row_mask"])
    w.forward(*args, row_weight=wt)
    dH, dE = w.backward(*args, grad=g, row_weight=wt, reuse=reuse, use_saved=use_saved, want_dH=want_dH,
                        want_dE=want_dE)
    torch.cuda.synchronize()
    return (None if dH is None else dH.clone()), (None if dE is None else dE.clone())


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("weighted", [False, True])
def test_reuse_gives_the_bits_of_the_full_backward(name, kw, weighted):
    d = _dev(W.custom_problem(**kw))
    wt = _weights(kw["R"], kw["seed"] + 100) if weighted else None
    w = Workspace(d["H"], d["E"], d["item_ids"], save_dh=True)
    g = torch.tensor([0.75], device="cuda")
    ref = _step(w, d, g, wt, reuse=False)
    got = _step(w, d, g, wt, reuse=True)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert torch.isfinite(ref[1].float()).all() and ref[1].abs().max().item() > 0


@pytest.mark.parametrize("name,kw", [CASES[1], CASES[3]], ids=[CASES[1][0], CASES[3][0]])
def test_reuse_single_outputs_and_recompute_path(name, kw):
    d = _dev(W.custom_problem(**kw))
    w = Workspace(d["H"], d["E"], d["item_ids"], save_dh=True)
    g = torch.tensor([-1.5], device="cuda")
    full = _step(w, d, g, None, reuse=False)
    # dE only, dH only (scaled dh_saved), and dH recomputed without dh_saved
    assert torch.equal(_step(w, d, g, None, reuse=True, want_dH=False)[1], full[1])
    assert torch.equal(_step(w, d, g, None, reuse=True, want_dE=False)[0], full[0])
    assert torch.equal(_step(w, d, g, None, reuse=True, use_saved=False)[0],
                       _step(w, d, g, None, reuse=False, use_saved=False)[0])


def test_reuse_after_a_forward_without_saved_dh():
    kw = CASES[1][1]
    d = _dev(W.custom_problem(**kw))
    w_ref = Workspace(d["H"], d["E"], d["item_ids"], save_dh=True)
    g = torch.tensor([1.0], device="cuda")
    ref = _step(w_ref, d, g, None, reuse=False)
    w = Workspace(d["H"], d["E"], d["item_ids"], save_dh=False)
    got = _step(w, d, g, None, reuse=True, use_saved=False)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_autograd_front_end_matches_the_explicit_calls():
    kw = CASES[0][1]
    d = _dev(W.custom_problem(**kw))
    w = Workspace(d["H"], d["E"], d["item_ids"], save_dh=True)
    g = torch.tensor([1.0], device="cuda")
    ref = _step(w, d, g, None, reuse=False)
    H = d["H"].clone().requires_grad_(True)
    E = d["E"].clone().requires_grad_(True)
    loss = cut_bce(H, E, d["row_offsets"], d["item_ids"], d["row_mask"])
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss.detach().reshape(1), w.loss)
    assert torch.equal(H.grad, ref[0]) and torch.equal(E.grad, ref[1])


def test_graph_replays_of_forward_and_reused_backward():
    kw = CASES[1][1]
    p = W.custom_problem(**kw)
    a = _dev(p)
    gen = torch.Generator().manual_seed(87)
    b = dict(a, H=(0.5 * torch.randn(p["H"].shape, generator=gen)).to(p["H"].dtype).cuda(),
             E=(0.5 * torch.randn(p["E"].shape, generator=gen)).to(p["E"].dtype).cuda(),
             row_mask=torch.ones_like(a["row_mask"]))
    w = Workspace(a["H"], a["E"], a["item_ids"], save_dh=True)
    g = torch.tensor([0.5], device="cuda")
    ref = _step(w, a, g, None, reuse=False)

    def capt():
        args = (a["H"], a["E"], a["row_offsets"], a["item_ids"], a["row_mask"])
        w.forward(*args)
        return w.backward(*args, grad=g, reuse=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capt()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdH, gdE = capt()
    torch.cuda.synchronize()
    for _ in range(3):
        _step(w, b, g, None, reuse=True)  # another mask and other inputs through the same workspace
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gdH, ref[0]) and torch.equal(gdE, ref[1])
