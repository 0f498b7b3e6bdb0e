"""ctypes binding of libcutbce.so (C ABI in include/cutbce.h).

Every function here only marshals arguments: tensors become device pointers, the current torch stream becomes
the hipStream_t, and status codes become exceptions. All computation happens in the HIP library. If the
library has not been built, the first call raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcutbce.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
_lock = threading.Lock()
_lib = None


class CutBCEError(RuntimeError):
    pass


class Problem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("vocab", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


EXPORTS = ["cutbce_workspace_size", "cutbce_forward", "cutbce_forward_noalloc", "cutbce_backward",
           "cutbce_backward_reuse", "cutbce_validate_targets",
           "cutbce_targets_to_csr", "cutbce_topk",
           "cutbce_profile_enable", "cutbce_profile_read", "cutbce_mfma_ceiling",
           "cutbce_mfma_ceiling_random", "cutbce_status_string",
           "cutbce_version"]


def lib():
    """Load libcutbce.so once; raise if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise CutBCEError(f"{LIB_PATH} is not built; run `python -m vocabulary_label_bce_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        P = ctypes.POINTER(Problem)
        L.cutbce_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
        L.cutbce_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.cutbce_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.cutbce_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.cutbce_backward_reuse.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.cutbce_validate_targets.argtypes = [P, vp, vp, vp, vp]
        L.cutbce_targets_to_csr.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int32, vp, vp, vp]
        L.cutbce_topk.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, sz, vp]
        L.cutbce_profile_enable.argtypes = [i32]
        L.cutbce_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32]
        L.cutbce_profile_enable.restype = i32
        L.cutbce_profile_read.restype = i32
        L.cutbce_mfma_ceiling.argtypes = [i32, i32, i32, vp, vp]
        L.cutbce_mfma_ceiling.restype = i32
        L.cutbce_mfma_ceiling_random.argtypes = [i32, i32, i32, vp, vp]
        L.cutbce_mfma_ceiling_random.restype = i32
        L.cutbce_status_string.argtypes = [i32]
        L.cutbce_status_string.restype = ctypes.c_char_p
        L.cutbce_version.restype = i32
        for f in ("cutbce_workspace_size", "cutbce_forward", "cutbce_forward_noalloc", "cutbce_backward",
                  "cutbce_backward_reuse", "cutbce_validate_targets",
                  "cutbce_targets_to_csr", "cutbce_topk"):
            getattr(L, f).restype = i32
        _lib = L
        return L


def _check(st: int):
    if st != 0:
        raise CutBCEError(f"cutbce status {st}: {lib().cutbce_status_string(st).decode()}")


def problem(R: int, V: int, nnz: int, D: int, dtype) -> Problem:
    dt = _DTYPES.get(dtype, dtype) if not isinstance(dtype, int) else dtype
    if dt not in (F32, BF16):
        raise CutBCEError(f"unsupported dtype {dtype}")
    return Problem(int(R), int(V), int(nnz), int(D), int(dt))


def workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().cutbce_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def problem_of(H, E, item_ids) -> Problem:
    return problem(H.shape[0], E.shape[0], item_ids.numel(), H.shape[1], H.dtype)


def alloc_workspace(p: Problem, device) -> torch.Tensor:
    return torch.empty(workspace_size(p), dtype=torch.uint8, device=device)


def forward(p: Problem, H, E, row_offsets, item_ids, row_mask, loss, row_loss, dh_saved, ws, stream=None,
            metrics=None, row_weight=None):
    """cutbce_forward on device tensors (outputs written in place; metrics: int32 [R, 4] or None;
    row_weight: float32 [R] or None)."""
    _check(lib().cutbce_forward(ctypes.byref(p), _ptr(H), _ptr(E), _ptr(row_offsets), _ptr(item_ids),
                                _ptr(row_mask), _ptr(row_weight), _ptr(loss), _ptr(row_loss), _ptr(dh_saved),
                                _ptr(metrics), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # CUTBCE_NOALLOC_SCRATCH_BYTES


def forward_noalloc(p: Problem, H, E, row_offsets, item_ids, row_mask, loss, row_loss, dh_saved, stream=None,
                    metrics=None, row_weight=None):
    """cutbce_forward_noalloc: cutbce_forward with the library's own per-GPU scratch array as workspace."""
    _check(lib().cutbce_forward_noalloc(ctypes.byref(p), _ptr(H), _ptr(E), _ptr(row_offsets), _ptr(item_ids),
                                        _ptr(row_mask), _ptr(row_weight), _ptr(loss), _ptr(row_loss),
                                        _ptr(dh_saved), _ptr(metrics), _stream(stream)))


def backward(p: Problem, H, E, row_offsets, item_ids, row_mask, grad_loss, dh_saved, dH, dE, ws, stream=None,
             row_weight=None, reuse=False):
    """cutbce_backward on device tensors (dH / dE overwritten in place; either may be None). reuse=True calls
    cutbce_backward_reuse: `ws` must hold what cutbce_forward left for these same inputs."""
    f = lib().cutbce_backward_reuse if reuse else lib().cutbce_backward
    _check(f(ctypes.byref(p), _ptr(H), _ptr(E), _ptr(row_offsets), _ptr(item_ids), _ptr(row_mask),
             _ptr(row_weight), _ptr(grad_loss), _ptr(dh_saved), _ptr(dH), _ptr(dE), _ptr(ws),
             ws.numel() if ws is not None else 0, _stream(stream)))


def topk(p: Problem, H, E, row_offsets, item_ids, row_mask, k: int, top_vals, top_ids, hits, ws, stream=None):
    """cutbce_topk on device tensors: top_vals float [R, k], top_ids int32 [R, k], hits int32 [R] or None."""
    _check(lib().cutbce_topk(ctypes.byref(p), _ptr(H), _ptr(E), _ptr(row_offsets), _ptr(item_ids), _ptr(row_mask),
                             int(k), _ptr(top_vals), _ptr(top_ids), _ptr(hits), _ptr(ws),
                             ws.numel() if ws is not None else 0, _stream(stream)))


def targets_to_csr(targets, pad_id: int, row_offsets, item_ids, stream=None):
    """cutbce_targets_to_csr: targets int32 [R, L] on the device -> row_offsets [R+1], item_ids [R*L] (in place)."""
    R, L = targets.shape
    _check(lib().cutbce_targets_to_csr(int(R), int(L), _ptr(targets), int(pad_id), _ptr(row_offsets),
                                       _ptr(item_ids), _stream(stream)))


def validate_targets(p: Problem, row_offsets, item_ids, bad, stream=None):
    _check(lib().cutbce_validate_targets(ctypes.byref(p), _ptr(row_offsets), _ptr(item_ids), _ptr(bad),
                                         _stream(stream)))


SWEEP_KINDS = ("rows_sweep", "items_sweep", "topk_sweep")


def profile_enable(on: bool = True):
    """Start (or stop) event timing of the sweep kernels inside the library."""
    _check(lib().cutbce_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kind: (total_ms, launches)} since the last enable/read; waits for the recorded events."""
    n = len(SWEEP_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().cutbce_profile_read(ms, cnt, n))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(SWEEP_KINDS)}


def mfma_ceiling(blocks: int, waves_per_block: int, iters: int, stamps, stream=None):
    """Enqueue the MFMA-only ceiling kernel; stamps: int64 device tensor of 4 * blocks * waves_per_block."""
    _check(lib().cutbce_mfma_ceiling(blocks, waves_per_block, iters, _ptr(stamps), _stream(stream)))


def mfma_ceiling_random(blocks: int, waves_per_block: int, iters: int, stamps, stream=None):
    """Enqueue the MFMA-only ceiling kernel on random operands that change from one MFMA to the next."""
    _check(lib().cutbce_mfma_ceiling_random(blocks, waves_per_block, iters, _ptr(stamps), _stream(stream)))
