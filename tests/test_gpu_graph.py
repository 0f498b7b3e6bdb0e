"""Graph capture of the forward + backward calls through the C ABI (torch.cuda.graph records a HIP graph on
ROCm). Every replay recomputes everything from the inputs: between replays an eager run of another problem of
the same shape overwrites the outputs and the workspace, and each replay must then give the eager results of
the captured problem bit for bit."""
import pytest
import torch

from vocabulary_label_bce_amd import workloads as W
from vocabulary_label_bce_amd.ops import Workspace

pytestmark = pytest.mark.gpu


def _args(p, H, E):
    return (H, E, p["row_offsets"].cuda(), p["item_ids"].cuda(), p["row_mask"].cuda())


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 256), ("bf16", 512)])
def test_graph_replays_match_eager(dtype, D):
    p = W.custom_problem(300, 5000, D, dtype=dtype, seed=41, h_std=0.3, e_std=0.3, pos_per_row=(1, 8),
                         mask_frac=0.2)
    a = _args(p, p["H"].cuda(), p["E"].cuda())
    # same positives and mask (so the same workspace size), other embeddings
    gen = torch.Generator().manual_seed(43)
    b = _args(p, (0.3 * torch.randn(p["H"].shape, generator=gen)).to(p["H"].dtype).cuda(),
              (0.3 * torch.randn(p["E"].shape, generator=gen)).to(p["E"].dtype).cuda())
    w = Workspace(a[0], a[1], a[3], want_row_loss=True, save_dh=True)
    g = torch.tensor([0.5], device="cuda")

    def step(x):
        w.forward(*x)
        return w.backward(*x, grad=g)

    dH, dE = step(a)
    torch.cuda.synchronize()
    ref = [w.loss.clone(), w.row_loss.clone(), dH.clone(), dE.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdH, gdE = step(a)
    torch.cuda.synchronize()

    for _ in range(3):
        step(b)  # eager work in between: other inputs through the same workspace and outputs
        torch.cuda.synchronize()
        assert not torch.equal(w.loss, ref[0])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(w.loss, ref[0])
        assert torch.equal(w.row_loss, ref[1])
        assert torch.equal(gdH, ref[2])
        assert torch.equal(gdE, ref[3])
