"""PyTorch front end: ``cut_bce`` is a differentiable full-vocabulary BCE whose forward and backward run in
libcutbce.so ("Cut Binary Cross Entropy", Listing 1 and the custom VJP of Section III-B).

PyTorch only allocates memory (inputs, outputs, the scratch workspace and the saved dH) and supplies the
stream; the library does all the arithmetic. Inputs must live on the GPU; there is no CPU path.
"""
from __future__ import annotations

import torch

from . import binding as B


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
    def forward(ctx, H, E, row_offsets, item_ids, row_mask):
        p = B.problem_of(H, E, item_ids)
        ws = B.alloc_workspace(p, H.device)
        loss = torch.empty(1, dtype=torch.float32, device=H.device)
        dh_saved = None
        if ctx.needs_input_grad[0]:
            dh_saved = torch.empty(H.shape, dtype=torch.float32, device=H.device)
        B.forward(p, H, E, row_offsets, item_ids, row_mask, loss, None, dh_saved, ws)
        ctx.save_for_backward(H, E, row_offsets, item_ids, row_mask, dh_saved)
        ctx.p = p
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        H, E, row_offsets, item_ids, row_mask, dh_saved = ctx.saved_tensors
        p = ctx.p
        g = g.reshape(1).to(dtype=torch.float32).contiguous()
        dH = torch.empty_like(H) if ctx.needs_input_grad[0] else None
        dE = torch.empty_like(E) if ctx.needs_input_grad[1] else None
        if dH is not None or dE is not None:
            ws = B.alloc_workspace(p, H.device)
            B.backward(p, H, E, row_offsets, item_ids, row_mask, g, dh_saved, dH, dE, ws)
        return dH, dE, None, None, None


def cut_bce(H, E, row_offsets, item_ids, row_mask):
    """Exact full-vocabulary BCE loss over logits H @ E^T, averaged over valid rows and all V items.

    H [R, D] and E [V, D] (float32 or bfloat16, on the GPU); positives of row r are
    item_ids[row_offsets[r]:row_offsets[r+1]] (any order, repeats count once); row_mask [R] marks valid rows.
    Returns a 0-d float32 tensor; gradients flow to H and E.
    """
    H, E, row_offsets, item_ids, row_mask = _prep(H, E, row_offsets, item_ids, row_mask)
    return _CutBCE.apply(H, E, row_offsets, item_ids, row_mask)


def dense_to_csr(targets, pad_id: int = -1):
    """Targets as a padded [B, N, L] (or [R, L]) id tensor -> (row_offsets, item_ids), dropping `pad_id`."""
    t = targets.reshape(-1, targets.shape[-1])
    keep = t != pad_id
    counts = keep.sum(1)
    row_offsets = torch.zeros(t.shape[0] + 1, dtype=torch.int32, device=t.device)
    row_offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return row_offsets, t[keep].to(torch.int32)


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

    def forward(self, H, E, row_offsets, item_ids, row_mask, stream=None):
        B.forward(self.p, H, E, row_offsets, item_ids, row_mask, self.loss, self.row_loss, self.dh_saved, self.ws,
                  stream, metrics=self.metrics)
        return self.loss

    def backward(self, H, E, row_offsets, item_ids, row_mask, grad=None, want_dH=True, want_dE=True,
                 use_saved=True, stream=None):
        g = self.grad if grad is None else grad
        B.backward(self.p, H, E, row_offsets, item_ids, row_mask, g, self.dh_saved if use_saved else None,
                   self.dH if want_dH else None, self.dE if want_dE else None, self.ws, stream)
        return (self.dH if want_dH else None), (self.dE if want_dE else None)
