"""PyTorch front end: ``cut_bce`` is a differentiable full-vocabulary BCE whose forward and backward run in
libcutbce.so ("Cut Binary Cross Entropy", Listing 1 and the custom VJP of Section III-B).

PyTorch only allocates memory (inputs, outputs, the scratch workspace and the saved dH) and supplies the
stream; the library does all the arithmetic. Inputs must live on the GPU; there is no CPU path.
"""
from __future__ import annotations

import torch

from . import binding as B


def _weights(row_weight, H):
    """float32 [R] row weights on H's device, or None."""
    if row_weight is None:
        return None
    w = row_weight.to(device=H.device, dtype=torch.float32).reshape(-1).contiguous()
    if w.numel() != H.shape[0]:
        raise ValueError("row_weight must have R entries")
    return w


def _prep(H, E, row_offsets, item_ids, row_mask):
    if not (H.is_cuda and E.is_cuda):
        raise ValueError("cut_bce runs on the GPU only: H and E must be device tensors")
    if H.dtype != E.dtype or H.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("H and E must both be float32 or both bfloat16")
    if H.dim() != 2 or E.dim() != 2 or H.shape[1] != E.shape[1]:
        raise ValueError("H must be [R, D] and E [V, D]")
    dev = H.device
    H = H.contiguous()
    E = E.contiguous()
    row_offsets = row_offsets.to(device=dev, dtype=torch.int32).contiguous()
    item_ids = item_ids.to(device=dev, dtype=torch.int32).contiguous()
    row_mask = row_mask.to(device=dev, dtype=torch.uint8).contiguous()
    if row_offsets.numel() != H.shape[0] + 1 or row_mask.numel() != H.shape[0]:
        raise ValueError("row_offsets must have R+1 entries and row_mask R entries")
    return H, E, row_offsets, item_ids, row_mask


class _CutBCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, E, row_offsets, item_ids, row_mask, row_weight):
        p = B.problem_of(H, E, item_ids)
        ws = B.alloc_workspace(p, H.device)
        loss = torch.empty(1, dtype=torch.float32, device=H.device)
        dh_saved = None
        if ctx.needs_input_grad[0]:
            dh_saved = torch.empty(H.shape, dtype=torch.float32, device=H.device)
        B.forward(p, H, E, row_offsets, item_ids, row_mask, loss, None, dh_saved, ws, row_weight=row_weight)
        ctx.save_for_backward(H, E, row_offsets, item_ids, row_mask, dh_saved, row_weight)
        ctx.p = p
        # the workspace keeps the forward's row preparation for the backward (cutbce_backward_reuse); autograd's
        # version check on the saved inputs rejects an in-place change of them in between
        ctx.ws = ws if (ctx.needs_input_grad[0] or ctx.needs_input_grad[1]) else None
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        H, E, row_offsets, item_ids, row_mask, dh_saved, row_weight = ctx.saved_tensors
        p = ctx.p
        g = g.reshape(1).to(dtype=torch.float32).contiguous()
        dH = torch.empty_like(H) if ctx.needs_input_grad[0] else None
        dE = torch.empty_like(E) if ctx.needs_input_grad[1] else None
        ws, ctx.ws = ctx.ws, None
        if (dH is not None or dE is not None) and ws is not None:
            B.backward(p, H, E, row_offsets, item_ids, row_mask, g, dh_saved, dH, dE, ws, row_weight=row_weight,
                       reuse=True)
        return dH, dE, None, None, None, None


def cut_bce(H, E, row_offsets, item_ids, row_mask, row_weight=None):
    """Exact full-vocabulary BCE loss over logits H @ E^T, averaged over valid rows and all V items.

    H [R, D] and E [V, D] (float32 or bfloat16, on the GPU); positives of row r are
    item_ids[row_offsets[r]:row_offsets[r+1]] (any order, repeats count once); row_mask [R] marks valid rows.
    row_weight [R] (optional, finite and >= 0): per-row weights; the loss becomes the weighted average
    sum_r w_r sum_v L / (W V) over valid rows, W = sum of their weights (no weights: W = number of valid rows).
    Returns a 0-d float32 tensor; gradients flow to H and E (not to the weights).
    """
    H, E, row_offsets, item_ids, row_mask = _prep(H, E, row_offsets, item_ids, row_mask)
    return _CutBCE.apply(H, E, row_offsets, item_ids, row_mask, _weights(row_weight, H))


def dense_to_csr(targets, pad_id: int = -1):
    """Padded targets [B, N, L] (or [R, L]) on the GPU -> (row_offsets [R+1], item_ids [R*L]) on the device
    (cutbce_targets_to_csr): slots equal to `pad_id` are dropped, order is kept; item_ids is capacity-sized and
    only its first row_offsets[R] entries are used. No host synchronisation."""
    if not targets.is_cuda:
        raise ValueError("dense_to_csr runs on the GPU only")
    rows = 1
    for n in targets.shape[:-1]:
        rows *= int(n)
    t = targets.reshape(rows, targets.shape[-1]).to(torch.int32).contiguous()
    R, L = t.shape
    row_offsets = torch.empty(R + 1, dtype=torch.int32, device=t.device)
    item_ids = torch.empty(max(R * L, 1), dtype=torch.int32, device=t.device)
    B.targets_to_csr(t, pad_id, row_offsets, item_ids)
    return row_offsets, item_ids


def cut_binary_cross_entropy(activations, embeddings, targets, weights=None, pad_id: int = -1):
    """The paper's Listing 1 call shape: activations [B, N, D], embeddings [V, D], targets [B, N, L] (ids, slots
    equal to `pad_id` are padding), weights [B, N] per position or None (all positions weigh 1).

    A position of weight 0 is padding: it is left out, and so are its targets. The others are averaged with
    their weights: loss = sum_pos w sum_v L / (sum_pos w * V). 0/1 weights give the plain average over the
    trained positions. Weights must be finite and >= 0 (not checked: that would read them back to the host).
    Returns the scalar loss; gradients flow to activations and embeddings.
    """
    B_, N = activations.shape[0], activations.shape[1]
    H = activations.reshape(B_ * N, activations.shape[-1])
    row_offsets, item_ids = dense_to_csr(targets, pad_id)
    if weights is None:
        mask = torch.ones(B_ * N, dtype=torch.uint8, device=H.device)
        return cut_bce(H, embeddings, row_offsets, item_ids, mask)
    w = weights.reshape(B_ * N).to(device=H.device)
    mask = (w != 0).to(torch.uint8)
    return cut_bce(H, embeddings, row_offsets, item_ids, mask, row_weight=w)


def topk(H, E, k: int = 8, row_offsets=None, item_ids=None, row_mask=None, ws=None):
    """Full-vocabulary top-k of the logits H @ E^T per row, without materialising them (k <= 8): returns
    (vals float32 [R, k], ids int32 [R, k], hits int32 [R] or None). With row_offsets / item_ids (CSR
    positives) `hits` counts each row's positives among its k items (Hit@k = mean of hits > 0)."""
    if not (H.is_cuda and E.is_cuda):
        raise ValueError("topk runs on the GPU only")
    R = H.shape[0]
    dev = H.device
    want_hits = row_offsets is not None
    if row_offsets is None:
        row_offsets = torch.zeros(R + 1, dtype=torch.int32, device=dev)
        item_ids = torch.zeros(1, dtype=torch.int32, device=dev)
    if row_mask is None:
        row_mask = torch.ones(R, dtype=torch.uint8, device=dev)
    H, E, row_offsets, item_ids, row_mask = _prep(H, E, row_offsets, item_ids, row_mask)
    p = B.problem_of(H, E, item_ids)
    if ws is None:
        ws = B.alloc_workspace(p, dev)
    vals = torch.empty(R, k, dtype=torch.float32, device=dev)
    ids = torch.empty(R, k, dtype=torch.int32, device=dev)
    hits = torch.empty(R, dtype=torch.int32, device=dev) if want_hits else None
    B.topk(p, H, E, row_offsets, item_ids, row_mask, k, vals, ids, hits, ws)
    return vals, ids, hits


class Workspace:
    """Reusable explicit-call wrapper: one workspace per problem shape, outputs allocated once."""

    def __init__(self, H, E, item_ids, want_row_loss=False, save_dh=True, want_metrics=False):
        self.p = B.problem_of(H, E, item_ids)
        dev = H.device
        self.ws = B.alloc_workspace(self.p, dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.row_loss = torch.empty(H.shape[0], dtype=torch.float32, device=dev) if want_row_loss else None
        self.dh_saved = torch.empty(H.shape, dtype=torch.float32, device=dev) if save_dh else None
        # Cut Metrics: TP, FP, FN, TN per row
        self.metrics = torch.empty(H.shape[0], 4, dtype=torch.int32, device=dev) if want_metrics else None
        self.grad = torch.ones(1, dtype=torch.float32, device=dev)
        self.dH = torch.empty_like(H)
        self.dE = torch.empty_like(E)

    def forward(self, H, E, row_offsets, item_ids, row_mask, stream=None, row_weight=None):
        B.forward(self.p, H, E, row_offsets, item_ids, row_mask, self.loss, self.row_loss, self.dh_saved, self.ws,
                  stream, metrics=self.metrics, row_weight=row_weight)
        return self.loss

    def backward(self, H, E, row_offsets, item_ids, row_mask, grad=None, want_dH=True, want_dE=True,
                 use_saved=True, stream=None, row_weight=None, reuse=False):
        """reuse=True: the previous call on this workspace was forward() with the same H, targets, mask and
        weights (cutbce_backward_reuse skips the row compaction and the H preparation)."""
        g = self.grad if grad is None else grad
        B.backward(self.p, H, E, row_offsets, item_ids, row_mask, g, self.dh_saved if use_saved else None,
                   self.dH if want_dH else None, self.dE if want_dE else None, self.ws, stream,
                   row_weight=row_weight, reuse=reuse)
        return (self.dH if want_dH else None), (self.dE if want_dE else None)
