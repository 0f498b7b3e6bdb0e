"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/cutbce.h declares, sizes its workspace without any [rows, V] term, and rejects bad arguments before
anything is enqueued (these paths make no HIP call, so fake device pointers are safe)."""
import ctypes
import os
import re

import pytest

from vocabulary_label_bce_amd import binding as B
from vocabulary_label_bce_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cutbce.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(cutbce_[a-z_]+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in cutbce.h but not exported"
    assert set(B.EXPORTS) == set(names)
    assert lib.cutbce_version() >= 200  # row_weight in cutbce_forward / cutbce_backward


def test_status_strings():
    lib = B.lib()
    for code in range(8):
        assert lib.cutbce_status_string(code)
    assert lib.cutbce_status_string(0) == b"ok"


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_workspace_has_no_rows_times_vocab_term(name):
    cfg = W.CONFIGS[name]
    p = B.problem(cfg.R, cfg.V, 40 * cfg.R, cfg.D, B.BF16 if cfg.dtype == "bf16" else B.F32)
    ws = B.workspace_size(p)
    # one re-laid-out copy of E plus O((R + V/256) * D) bookkeeping, never R*V
    esz = 2 if cfg.dtype == "bf16" else 4
    assert ws < cfg.V * cfg.D * esz * 1.2 + 1100 * 256 * cfg.D * 4 * 1.5 + 64 * cfg.R * cfg.D + (1 << 26)
    assert ws < 0.5 * W.dense_logits_bytes(cfg.R, cfg.V) or cfg.R * cfg.V < 1e7


def _call_forward(p, H=16, E=16, ro=16, ids=16, mask=16, loss=16, ws=256, ws_bytes=None, metrics=None,
                  weight=None):
    lib = B.lib()
    if ws_bytes is None:
        try:
            ws_bytes = B.workspace_size(p)
        except B.CutBCEError:
            ws_bytes = 1 << 40
    vp = ctypes.c_void_p
    return lib.cutbce_forward(ctypes.byref(p), vp(H), vp(E), vp(ro), vp(ids), vp(mask),
                              vp(weight) if weight else None, vp(loss), None, None,
                              vp(metrics) if metrics else None, vp(ws), ws_bytes, None)


FAKE = 1 << 20  # aligned, never dereferenced: every case below fails a host check first


def test_forward_rejects_bad_arguments():
    good = B.problem(64, 4096, 100, 64, B.BF16)
    assert _call_forward(good, H=0, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 1  # NULL
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=0, ws=FAKE) == 1
    assert _call_forward(good, H=FAKE + 2, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 4  # align
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE,
                         ws_bytes=1024) == 5  # workspace
    bad_dim = B.problem(64, 4096, 100, 96, B.BF16)
    assert _call_forward(bad_dim, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 6
    bad_f32 = B.problem(64, 4096, 100, 512, B.F32)
    assert _call_forward(bad_f32, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 6
    bad_shape = B.Problem(0, 4096, 100, 64, 1)
    assert _call_forward(bad_shape, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 2
    bad_dtype = B.Problem(64, 4096, 100, 64, 7)
    assert _call_forward(bad_dtype, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 3
    neg_nnz = B.Problem(64, 4096, -1, 64, 1)
    assert _call_forward(neg_nnz, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE) == 2
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE,
                         metrics=FAKE + 2) == 4  # misaligned metrics
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE,
                         weight=FAKE + 2) == 4  # misaligned row weights
    # nnz > 0 needs item_ids
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=0, mask=FAKE, loss=FAKE, ws=FAKE) == 1
    # the workspace must be 256-byte aligned (16 is not enough)
    assert _call_forward(good, H=FAKE, E=FAKE, ro=FAKE, ids=FAKE, mask=FAKE, loss=FAKE, ws=FAKE + 128) == 4


def test_size_limits_at_their_boundaries():
    """R and V up to 2^31 - 1025 are accepted (the workspace size is computed), one more is SHAPE; nnz up to
    2^31 - 1."""
    lim = (1 << 31) - 1025
    sz = ctypes.c_size_t()
    lib = B.lib()
    for R, V, nnz in [(lim, 4096, 100), (64, lim, 100), (64, 4096, (1 << 31) - 1)]:
        assert lib.cutbce_workspace_size(ctypes.byref(B.Problem(R, V, nnz, 64, 1)), ctypes.byref(sz)) == 0
        assert sz.value > 0
    for R, V, nnz in [(lim + 1, 4096, 100), (64, lim + 1, 100), (64, 4096, 1 << 31)]:
        assert lib.cutbce_workspace_size(ctypes.byref(B.Problem(R, V, nnz, 64, 1)), ctypes.byref(sz)) == 2


def test_backward_and_validate_reject_bad_arguments():
    lib = B.lib()
    p = B.problem(64, 4096, 100, 128, B.BF16)
    vp = ctypes.c_void_p
    ws = B.workspace_size(p)
    # grad_loss NULL
    assert lib.cutbce_backward(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, None,
                               None, vp(FAKE), vp(FAKE), vp(FAKE), ws, None) == 1
    # misaligned dE
    assert lib.cutbce_backward(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE),
                               None, vp(FAKE), vp(FAKE + 4), vp(FAKE), ws, None) == 4
    # misaligned row weights
    assert lib.cutbce_backward(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE + 2),
                               vp(FAKE), None, vp(FAKE), vp(FAKE), vp(FAKE), ws, None) == 4
    # workspace too small
    assert lib.cutbce_backward(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE),
                               None, vp(FAKE), vp(FAKE), vp(FAKE), ws - 1, None) == 5
    assert lib.cutbce_validate_targets(ctypes.byref(p), None, vp(FAKE), vp(FAKE), None) == 1
    assert lib.cutbce_validate_targets(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE + 2), None) == 4
    n = ctypes.c_size_t(0)
    assert lib.cutbce_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.cutbce_workspace_size(ctypes.byref(p), None) == 1


def test_topk_rejects_bad_arguments():
    lib = B.lib()
    vp = ctypes.c_void_p
    p = B.problem(64, 4096, 100, 128, B.BF16)
    ws = B.workspace_size(p)
    args = lambda k, vals=FAKE, ids=FAKE: (ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), k,
                                           vp(vals) if vals else None, vp(ids) if ids else None, None, vp(FAKE), ws,
                                           None)
    assert lib.cutbce_topk(*args(0)) == 2
    assert lib.cutbce_topk(*args(9)) == 2
    assert lib.cutbce_topk(*args(8, vals=0)) == 1
    assert lib.cutbce_topk(*args(8, ids=FAKE + 2)) == 4
    small = B.problem(64, 5, 100, 128, B.BF16)
    assert lib.cutbce_topk(ctypes.byref(small), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 6, vp(FAKE),
                           vp(FAKE), None, vp(FAKE), B.workspace_size(small), None) == 2  # k > V


def test_targets_to_csr_rejects_bad_arguments():
    lib = B.lib()
    vp = ctypes.c_void_p
    assert lib.cutbce_targets_to_csr(0, 4, vp(FAKE), -1, vp(FAKE), vp(FAKE), None) == 2  # no rows
    assert lib.cutbce_targets_to_csr(8, -1, vp(FAKE), -1, vp(FAKE), vp(FAKE), None) == 2  # negative slots
    assert lib.cutbce_targets_to_csr(1 << 20, 1 << 12, vp(FAKE), -1, vp(FAKE), vp(FAKE), None) == 2  # R*L >= 2^31
    assert lib.cutbce_targets_to_csr(8, 4, None, -1, vp(FAKE), vp(FAKE), None) == 1
    assert lib.cutbce_targets_to_csr(8, 4, vp(FAKE), -1, None, vp(FAKE), None) == 1
    assert lib.cutbce_targets_to_csr(8, 4, vp(FAKE + 2), -1, vp(FAKE), vp(FAKE), None) == 4


def test_library_source_never_allocates_device_memory():
    csrc = os.path.join(ROOT, "vocabulary_label_bce_amd", "csrc")
    for f in os.listdir(csrc):
        txt = open(os.path.join(csrc, f)).read()
        assert "hipMalloc" not in txt and "hipFree(" not in txt, f


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No CPU fallback: with libcutbce.so absent the binding raises before any computation."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libcutbce.so"))
    with pytest.raises(B.CutBCEError, match="not built"):
        B.lib()
    with pytest.raises(B.CutBCEError):
        B.workspace_size(B.problem(64, 4096, 100, 64, B.BF16))


def test_product_modules_never_import_the_oracle():
    import ast
    import os

    pkg = os.path.join(os.path.dirname(__file__), "..", "vocabulary_label_bce_amd")
    for name in os.listdir(pkg):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_mfma_ceiling_rejects_bad_arguments():
    L = B.lib()
    assert L.cutbce_mfma_ceiling(0, 8, 10, 8, None) == 2       # no workgroups
    assert L.cutbce_mfma_ceiling(1, 17, 10, 8, None) == 2      # more than 16 waves
    assert L.cutbce_mfma_ceiling(1, 8, 0, 8, None) == 2        # no iterations
    assert L.cutbce_mfma_ceiling(1, 8, 10, None, None) == 1    # no stamp buffer
    assert L.cutbce_mfma_ceiling(1, 8, 10, 12, None) == 4      # misaligned stamp buffer
    assert L.cutbce_mfma_ceiling_random(0, 8, 10, 8, None) == 2
    assert L.cutbce_mfma_ceiling_random(1, 17, 10, 8, None) == 2
    assert L.cutbce_mfma_ceiling_random(1, 8, 0, 8, None) == 2
    assert L.cutbce_mfma_ceiling_random(1, 8, 10, None, None) == 1
    assert L.cutbce_mfma_ceiling_random(1, 8, 10, 12, None) == 4


def test_noalloc_forward_rejects_problems_beyond_its_scratch_before_any_hip_call():
    """cutbce_forward_noalloc checks the problem and its workspace size against the library's scratch array
    before it touches the device (fake pointers are never dereferenced)."""
    lib = B.lib()
    vp = ctypes.c_void_p
    big = B.problem(25600, 876000, 70000, 128, B.BF16)
    assert B.workspace_size(big) > B.NOALLOC_SCRATCH_BYTES
    st = lib.cutbce_forward_noalloc(ctypes.byref(big), vp(16), vp(16), vp(16), vp(16), vp(16), None, vp(16), None,
                                    None, None, None)
    assert st == 5  # CUTBCE_ERR_WORKSPACE
    bad = B.problem(0, 100, 0, 128, B.BF16)
    assert lib.cutbce_forward_noalloc(ctypes.byref(bad), vp(16), vp(16), vp(16), vp(16), vp(16), None, vp(16), None,
                                      None, None, None) == 2  # CUTBCE_ERR_SHAPE
