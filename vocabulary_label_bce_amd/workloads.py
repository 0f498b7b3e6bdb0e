"""Seeded synthetic inputs for the fused full-vocabulary BCE.

This module only draws inputs: hidden states H [R, D], item embeddings E [V, D], the positive ids of every
row in CSR form (row_offsets [R+1], item_ids [nnz]) and the row mask [R]. It holds none of the loss or
gradient arithmetic, so both the GPU library's tests and the float64 oracle can consume what it makes.

The shapes follow the paper's workloads ("Cut Binary Cross Entropy", Section IV-A mini-benchmark: activations
and embeddings drawn from a normal distribution, positive ids drawn over [0, V); Section III-E / IV-B:
SASRec-style sequences of at most N positions, left-padded, L next items per position, V = 876,939 items in
Yambda). The Yambda dataset itself is not used: the SASRec-shaped configuration stands in for it.

Recipe (the same for every configuration):
  * H and E: float32 normal draws from a seeded ``torch.Generator`` on the generating device, scaled by the
    configured standard deviation, then rounded to bfloat16 by round-to-nearest-even when the configuration
    is bf16. The portable variant (make_dense_portable) draws them with NumPy's PCG64 instead, so that the
    values do not depend on the host; the full-size parity tests use it with stored reference losses.
  * positives: per valid row a count, then that many *distinct* ids, uniform or from a bounded Zipf law over
    ranks 1..V (id = rank - 1, so id 0 is the hottest item); ids are stored sorted per row.
  * mask: 1 = position is trained, 0 = padding. Masked rows get no positives.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["WorkloadConfig", "CONFIGS", "make_problem", "zipf_sampler", "dense_logits_bytes"]


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    B: int
    N: int
    D: int
    V: int
    dtype: str            # "f32" or "bf16"
    h_std: float          # std of H draws (before the optional 1/sqrt(D))
    h_over_sqrt_d: bool   # H ~ N(0,1)/sqrt(D) when True
    e_std: float
    pos_count: tuple      # ("fixed", k) | ("uniform", lo, hi) | ("one_plus_poisson", lam)
    pos_ids: tuple        # ("uniform",) | ("zipf", s)
    mask: tuple           # ("random_frac", f) | ("trailing", n_masked) | ("left_pad", lo, hi) | ("none",)
    seed: int

    @property
    def R(self) -> int:
        return self.B * self.N


CONFIGS = {
    # Tiny CPU-checkable case: fp32, 3 distinct uniform positives per valid row, 10% of rows masked.
    "tiny": WorkloadConfig("tiny", 4, 16, 64, 4096, "f32", 0.1, False, 0.1,
                           ("fixed", 3), ("uniform",), ("random_frac", 0.1), 1001),
    # 6400 rows, V = 100k, bf16, 1-8 Zipf(1.1) positives, last 40 of 200 positions masked.
    "v100k": WorkloadConfig("v100k", 32, 200, 64, 100_000, "bf16", 1.0, True, 0.05,
                            ("uniform", 1, 8), ("zipf", 1.1), ("trailing", 40), 1002),
    # SASRec-shaped: 25.6k rows, V = 876k, D = 128, 1+Poisson(4) Zipf(1.05) positives, left padding.
    "sasrec876k": WorkloadConfig("sasrec876k", 128, 200, 128, 876_000, "bf16", 1.0, True, 0.02,
                                 ("one_plus_poisson", 4.0), ("zipf", 1.05), ("left_pad", 20, 200), 1003),
    # Max catalog: V = 10M, D = 256, 1-4 uniform positives, no padding.
    "catalog10m": WorkloadConfig("catalog10m", 16, 256, 256, 10_000_000, "bf16", 1.0, True, 0.02,
                                 ("uniform", 1, 4), ("uniform",), ("none",), 1004),
    # Positive-dense: D = 512, 64-256 Zipf(0.8) positives per row, 5% rows masked.
    "posdense": WorkloadConfig("posdense", 64, 64, 512, 262_144, "bf16", 1.0, True, 0.02,
                               ("uniform", 64, 256), ("zipf", 0.8), ("random_frac", 0.05), 1005),
}
CONFIG_ORDER = ["tiny", "v100k", "sasrec876k", "catalog10m", "posdense"]


def dense_logits_bytes(rows: int, vocab: int, bytes_per_elem: int = 4) -> int:
    """Size of a materialised [rows, V] logits buffer (Section I-A of the paper sizes it as B*N*V*4 bytes)."""
    return rows * vocab * bytes_per_elem


class zipf_sampler:
    """Bounded Zipf law over ranks 1..V with P(k) proportional to k^-s, sampled by inverse CDF (id = k-1)."""

    def __init__(self, V: int, s: float):
        w = np.arange(1, V + 1, dtype=np.float64) ** (-float(s))
        cdf = np.cumsum(w)
        self.cdf = cdf / cdf[-1]
        self.V = V

    def __call__(self, rng: np.random.Generator, n: int) -> np.ndarray:
        u = rng.random(n)
        return np.minimum(np.searchsorted(self.cdf, u, side="right"), self.V - 1).astype(np.int64)


def _mask(cfg: WorkloadConfig, rng: np.random.Generator) -> np.ndarray:
    R, B, N = cfg.R, cfg.B, cfg.N
    kind = cfg.mask[0]
    m = np.ones(R, dtype=np.uint8)
    if kind == "none":
        pass
    elif kind == "random_frac":
        n_masked = int(round(cfg.mask[1] * R))
        m[rng.choice(R, size=n_masked, replace=False)] = 0
    elif kind == "trailing":
        k = cfg.mask[1]
        m.reshape(B, N)[:, N - k:] = 0
    elif kind == "left_pad":
        lo, hi = cfg.mask[1], cfg.mask[2]
        lens = rng.integers(lo, hi + 1, size=B)
        mm = m.reshape(B, N)
        for b in range(B):
            mm[b, : N - lens[b]] = 0
    else:
        raise ValueError(kind)
    return m


def _counts(cfg: WorkloadConfig, rng: np.random.Generator, n: int) -> np.ndarray:
    kind = cfg.pos_count[0]
    if kind == "fixed":
        c = np.full(n, cfg.pos_count[1], dtype=np.int64)
    elif kind == "uniform":
        c = rng.integers(cfg.pos_count[1], cfg.pos_count[2] + 1, size=n)
    elif kind == "one_plus_poisson":
        c = 1 + rng.poisson(cfg.pos_count[1], size=n)
    else:
        raise ValueError(kind)
    return np.minimum(c, cfg.V).astype(np.int64)


def _distinct_ids(draw, rng, count: int) -> np.ndarray:
    """`count` distinct ids from `draw`, by rejection, returned sorted."""
    got: list = []
    seen: set = set()
    while len(got) < count:
        for x in draw(rng, max(2 * (count - len(got)), 8)).tolist():
            if x not in seen:
                seen.add(x)
                got.append(x)
                if len(got) == count:
                    break
    return np.sort(np.asarray(got, dtype=np.int64))


def make_targets(cfg: WorkloadConfig, seed: int | None = None):
    """Row mask and CSR positives (numpy int32/uint8) for a configuration."""
    seed = cfg.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    s_mask, s_cnt, s_ids = ss.spawn(3)
    mask = _mask(cfg, np.random.Generator(np.random.PCG64(s_mask)))
    valid = np.flatnonzero(mask)
    counts = np.zeros(cfg.R, dtype=np.int64)
    counts[valid] = _counts(cfg, np.random.Generator(np.random.PCG64(s_cnt)), valid.size)
    rng = np.random.Generator(np.random.PCG64(s_ids))
    if cfg.pos_ids[0] == "uniform":
        V = cfg.V

        def draw(g, n):
            return g.integers(0, V, size=n)
    else:
        draw = zipf_sampler(cfg.V, cfg.pos_ids[1])
    ids = [_distinct_ids(draw, rng, int(counts[r])) for r in valid]
    row_offsets = np.zeros(cfg.R + 1, dtype=np.int64)
    row_offsets[1:] = np.cumsum(counts)
    item_ids = np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)
    return mask, row_offsets.astype(np.int32), item_ids.astype(np.int32)


def make_dense_portable(cfg: WorkloadConfig, seed: int | None = None):
    """H [R, D] and E [V, D] on the CPU from NumPy's PCG64 (float32 standard normals by the ziggurat method,
    scaled, then rounded to bfloat16 when the configuration is bf16): the same values on any host, so values
    computed once from them (stored reference losses) stay valid wherever the inputs are drawn again."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919])))
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    h_std = cfg.h_std / math.sqrt(cfg.D) if cfg.h_over_sqrt_d else cfg.h_std
    H = (torch.from_numpy(rng.standard_normal((cfg.R, cfg.D), dtype=np.float32)) * h_std).to(tdt)
    E = torch.empty(cfg.V, cfg.D, dtype=tdt)
    slab = max(1, (1 << 26) // cfg.D)
    for v0 in range(0, cfg.V, slab):
        v1 = min(cfg.V, v0 + slab)
        E[v0:v1] = (torch.from_numpy(rng.standard_normal((v1 - v0, cfg.D), dtype=np.float32)) * cfg.e_std).to(tdt)
    return H, E


def make_dense(cfg: WorkloadConfig, seed: int | None = None, device: str | torch.device = "cpu"):
    """H [R, D] and E [V, D] drawn on `device` (torch dtypes float32 or bfloat16)."""
    seed = cfg.seed if seed is None else seed
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed * 7919 + 17)
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    h_std = cfg.h_std / math.sqrt(cfg.D) if cfg.h_over_sqrt_d else cfg.h_std
    H = (torch.randn(cfg.R, cfg.D, generator=g, device=dev, dtype=torch.float32) * h_std).to(tdt)
    # E can be large (5 GB at V = 10M, D = 256): draw it in slabs to bound the float32 temporary.
    E = torch.empty(cfg.V, cfg.D, device=dev, dtype=tdt)
    slab = max(1, (1 << 26) // cfg.D)
    for v0 in range(0, cfg.V, slab):
        v1 = min(cfg.V, v0 + slab)
        E[v0:v1] = (torch.randn(v1 - v0, cfg.D, generator=g, device=dev, dtype=torch.float32) * cfg.e_std).to(tdt)
    return H, E


def make_problem(name_or_cfg, seed: int | None = None, device="cpu", portable: bool = False):
    """Full problem as a dict of torch tensors on `device` plus the config. portable: H and E from
    make_dense_portable (host-independent values) instead of torch's generator on `device`."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    mask, ro, ids = make_targets(cfg, seed)
    if portable:
        H, E = make_dense_portable(cfg, seed)
        H, E = H.to(device), E.to(device)
    else:
        H, E = make_dense(cfg, seed, device)
    dev = torch.device(device)
    return dict(
        cfg=cfg,
        H=H,
        E=E,
        row_offsets=torch.from_numpy(ro).to(dev),
        item_ids=torch.from_numpy(ids).to(dev),
        row_mask=torch.from_numpy(mask).to(dev),
    )


def custom_problem(R, V, D, dtype="bf16", seed=0, h_std=1.0, e_std=1.0, pos_per_row=(1, 4),
                   mask_frac=0.0, dup_frac=0.0, device="cpu", zipf_s=None, sort_ids=True):
    """Small ad-hoc problem for edge cases (ragged sizes, duplicates, unsorted ids, planted values)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    mask = (rng.random(R) >= mask_frac).astype(np.uint8)
    counts = np.where(mask == 1, rng.integers(pos_per_row[0], pos_per_row[1] + 1, size=R), 0)
    counts = np.minimum(counts, V)
    draw = zipf_sampler(V, zipf_s) if zipf_s else (lambda g, n: g.integers(0, V, size=n))
    rows = []
    for r in range(R):
        ids = _distinct_ids(draw, rng, int(counts[r])) if counts[r] else np.zeros(0, np.int64)
        if dup_frac > 0 and ids.size:
            nd = int(np.ceil(dup_frac * ids.size))
            ids = np.concatenate([ids, rng.choice(ids, size=nd)])
        if sort_ids:
            ids = np.sort(ids)
        else:
            ids = rng.permutation(ids)
        rows.append(ids)
    ro = np.zeros(R + 1, dtype=np.int64)
    ro[1:] = np.cumsum([x.size for x in rows])
    item_ids = np.concatenate(rows) if R else np.zeros(0, np.int64)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    H = (torch.randn(R, D, generator=g) * h_std).to(tdt)
    E = (torch.randn(V, D, generator=g) * e_std).to(tdt)
    dev = torch.device(device)
    return dict(H=H.to(dev), E=E.to(dev),
                row_offsets=torch.from_numpy(ro.astype(np.int32)).to(dev),
                item_ids=torch.from_numpy(item_ids.astype(np.int32)).to(dev),
                row_mask=torch.from_numpy(mask).to(dev))
