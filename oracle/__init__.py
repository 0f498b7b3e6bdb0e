"""TEST INFRASTRUCTURE: float64 CPU oracle for the fused full-vocabulary BCE loss and gradients.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import this package.
It shares no code with the GPU library (``vocabulary_label_bce_amd``) and never imports it.

The arithmetic lives in ``cutbce_oracle.c`` (plain C, float64, OpenMP over rows/items); this module only
compiles it with gcc and marshals arrays. See the header of the C file for the equations it follows
("Cut Binary Cross Entropy", Section III-A Eq. (1)-(3), Section III-B Eq. (4), the Cut Metrics of
Section III-D and the full-vocabulary top-k / Hit@k evaluation of Section III-E).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cutbce_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_lock = threading.Lock()
_libs: dict = {}

ERRORS = {0: "ok", 1: "bad shape", 2: "bad ids/offsets", 3: "out of memory"}


def lib_path(plant: int = 0) -> str:
    return os.path.join(_BUILD, f"liboracle{'' if plant == 0 else f'_plant{plant}'}.so")


def build(plant: int = 0, force: bool = False) -> str:
    """Compile the oracle (optionally with a planted mistake, for pin-strength tests) and return its path."""
    out = lib_path(plant)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    os.makedirs(_BUILD, exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    # -std=c99 keeps floating-point contraction off: every product and sum is rounded as written
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99", f"-DORACLE_PLANT={plant}",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, out)
    return out


def _load(plant: int = 0):
    with _lock:
        if plant in _libs:
            return _libs[plant]
        lib = ctypes.CDLL(build(plant))
        i64, i32, f64, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.oracle_rows.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, f64, i64, vp, vp, vp]
        lib.oracle_items.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, f64, i64, vp, vp]
        lib.oracle_full.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, f64, vp, vp, vp, vp]
        lib.oracle_metrics.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, f64, i64, vp, vp]
        lib.oracle_topk.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp]
        for f in (lib.oracle_rows, lib.oracle_items, lib.oracle_full, lib.oracle_metrics, lib.oracle_topk,
                  lib.oracle_num_threads):
            f.restype = ctypes.c_int
        _libs[plant] = lib
        return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _dense(x):
    """(contiguous numpy array, dtype code): float32 -> 0, bfloat16 (as uint16 bits) -> 1."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), 1
        if x.dtype == torch.float32:
            return np.ascontiguousarray(x.numpy()), 0
        raise TypeError(f"oracle takes float32 or bfloat16, got {x.dtype}")
    x = np.asarray(x)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    raise TypeError(f"oracle takes float32 or bfloat16 bits (uint16), got {x.dtype}")


def _ints(x, dt):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x).astype(dt, copy=False))


def _prep(H, E, row_offsets, item_ids, row_mask):
    h, dt_h = _dense(H)
    e, dt_e = _dense(E)
    if dt_h != dt_e:
        raise TypeError("H and E must share a dtype")
    R, D = h.shape
    V, D2 = e.shape
    if D != D2:
        raise ValueError("H and E disagree on D")
    ro = _ints(row_offsets, np.int32)
    ids = _ints(item_ids, np.int32)
    if ids.size == 0:
        ids = np.zeros(1, np.int32)
    m = _ints(row_mask, np.uint8)
    return h, e, dt_h, R, V, D, ro, ids, m


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _weights(row_weight, R):
    """float64 [R] row weights, or None (every valid row weighs 1)."""
    if row_weight is None:
        return None
    if hasattr(row_weight, "detach"):
        row_weight = row_weight.detach().cpu().double().numpy()
    w = np.ascontiguousarray(np.asarray(row_weight, dtype=np.float64))
    if w.shape != (R,):
        raise ValueError(f"row_weight must have shape ({R},), got {w.shape}")
    return w


def _check(st):
    if st != 0:
        raise ValueError(f"oracle rejected the input: {ERRORS.get(st, st)}")


def full(H, E, row_offsets, item_ids, row_mask, g: float = 1.0, grads: bool = True, plant: int = 0,
         row_weight=None):
    """Loss, per-row losses (unweighted) and (optionally) dH [R, D], dE [V, D], all float64 numpy.
    row_weight: optional [R] weights of the rows (the weighted average of the C file's header)."""
    h, e, dt, R, V, D, ro, ids, m = _prep(H, E, row_offsets, item_ids, row_mask)
    w = _weights(row_weight, R)
    loss = np.zeros(1, np.float64)
    rl = np.zeros(R, np.float64)
    dH = np.zeros((R, D), np.float64) if grads else None
    dE = np.zeros((V, D), np.float64) if grads else None
    st = _load(plant).oracle_full(R, V, D, dt, _ptr(h), _ptr(e), _ptr(ro), _ptr(ids), _ptr(m),
                                  _ptr(w) if w is not None else None, float(g),
                                  _ptr(loss), _ptr(rl), _ptr(dH) if grads else None, _ptr(dE) if grads else None)
    _check(st)
    return dict(loss=float(loss[0]), row_loss=rl, dH=dH, dE=dE)


def rows(H, E, row_offsets, item_ids, row_mask, rows, g: float = 1.0, grads: bool = True, plant: int = 0,
         row_weight=None):
    """Per-row loss (unnormalised) and dH rows for the listed rows only (s uses all valid rows)."""
    h, e, dt, R, V, D, ro, ids, m = _prep(H, E, row_offsets, item_ids, row_mask)
    w = _weights(row_weight, R)
    rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    rl = np.zeros(rr.size, np.float64)
    dH = np.zeros((rr.size, D), np.float64) if grads else None
    st = _load(plant).oracle_rows(R, V, D, dt, _ptr(h), _ptr(e), _ptr(ro), _ptr(ids), _ptr(m),
                                  _ptr(w) if w is not None else None, float(g),
                                  rr.size, _ptr(rr), _ptr(rl), _ptr(dH) if grads else None)
    _check(st)
    return dict(row_loss=rl, dH=dH)


def items(H, E, row_offsets, item_ids, row_mask, items, g: float = 1.0, plant: int = 0, row_weight=None):
    """dE rows for the listed items only."""
    h, e, dt, R, V, D, ro, ids, m = _prep(H, E, row_offsets, item_ids, row_mask)
    w = _weights(row_weight, R)
    it = np.ascontiguousarray(np.asarray(items, dtype=np.int64))
    dE = np.zeros((it.size, D), np.float64)
    st = _load(plant).oracle_items(R, V, D, dt, _ptr(h), _ptr(e), _ptr(ro), _ptr(ids), _ptr(m),
                                   _ptr(w) if w is not None else None, float(g),
                                   it.size, _ptr(it), _ptr(dE))
    _check(st)
    return dict(dE=dE)


def metrics(H, E, row_offsets, item_ids, row_mask, rows=None, eps: float = 0.0, plant: int = 0):
    """Cut Metrics per row: int64 [n, 5] = TP, FP, FN, TN (prediction z > 0) and #{v : |z| <= eps}.
    All rows when `rows` is None; masked rows give zeros."""
    h, e, dt, R, V, D, ro, ids, m = _prep(H, E, row_offsets, item_ids, row_mask)
    if rows is None:
        rr, n, rp = None, R, None
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n, rp = rr.size, _ptr(rr)
    out = np.zeros((n, 5), np.int64)
    st = _load(plant).oracle_metrics(R, V, D, dt, _ptr(h), _ptr(e), _ptr(ro), _ptr(ids), _ptr(m), float(eps),
                                     n, rp, _ptr(out))
    _check(st)
    return out


def topk(H, E, row_offsets, item_ids, row_mask, k: int, rows=None, plant: int = 0):
    """Full-vocabulary top-k per row (all rows when `rows` is None): dict(ids int64 [n, k], vals float64 [n, k],
    hits int64 [n]) -- the k largest logits, ties by smaller item id; hits = how many of them are positives.
    Masked rows: ids -1, vals -inf, hits 0."""
    h, e, dt, R, V, D, ro, ids, m = _prep(H, E, row_offsets, item_ids, row_mask)
    if rows is None:
        n, rp = R, None
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n, rp = rr.size, _ptr(rr)
    oid = np.zeros((n, k), np.int64)
    oval = np.zeros((n, k), np.float64)
    hits = np.zeros(n, np.int64)
    st = _load(plant).oracle_topk(R, V, D, dt, _ptr(h), _ptr(e), _ptr(ro), _ptr(ids), _ptr(m), int(k), n, rp,
                                  _ptr(oid), _ptr(oval), _ptr(hits))
    _check(st)
    return dict(ids=oid, vals=oval, hits=hits)


def targets_to_csr(targets, pad_id: int = -1):
    """Dense padded targets [..., L] -> (row_offsets int32 [R+1], item_ids int32 [nnz]): the definition written
    out (the [B, N, L] target slots of the paper's Listing 1; a slot equal to pad_id is padding). Row r keeps
    its non-pad slots in slot order; rows follow in order."""
    t = np.asarray(targets.cpu().numpy() if hasattr(targets, "cpu") else targets)
    t = t.reshape(int(np.prod(t.shape[:-1])), t.shape[-1]) if t.ndim >= 2 else t.reshape(1, -1)
    offsets = [0]
    ids = []
    for row in t:
        kept = [int(x) for x in row if int(x) != pad_id]
        ids.extend(kept)
        offsets.append(offsets[-1] + len(kept))
    return np.asarray(offsets, np.int32), np.asarray(ids, np.int32)
