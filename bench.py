#!/usr/bin/env python3
"""Benchmark of the fused full-vocabulary BCE (CutBCE hot path) on one MI355X.

One step = cutbce_forward (loss, plus the saved dH) + cutbce_backward_reuse (dH and dE, reusing the forward's row
preparation) on the same inputs, i.e. the loss + gradient of "Cut Binary Cross Entropy" Section IV-A's isolated
mini-benchmark. Inputs are synthetic,
drawn on the GPU before the timed region (default workload: the SASRec-shaped 128 x 200 rows, D = 128,
V = 876,000, bf16).

Credited work per step: 8 * R_v * V * D flops (2 for the forward logits, 6 for the backward's recomputed logits,
dH and dE), R_v = valid rows. Padding rows, padding items and any extra recomputation are not credited.

Prints one JSON line. The CPU baseline times the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sasrec876k")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--topk", type=int, default=0,
                    help="instead of fwd+bwd, time full-vocabulary top-k scoring (cutbce_topk) of every valid row")
    ap.add_argument("--metrics", action="store_true",
                    help="also count the Cut Metrics (TP/FP/FN/TN per row) in the forward sweep")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain elementwise copy (torch.neg) of this many MiB three "
                         "times: the known-size reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def cpu_baseline(prob, R_v, target_s):
    """Time the float64 oracle on a seeded sample: whole-vocabulary rows (loss + dH) and whole-row items (dE)."""
    import numpy as np

    import oracle

    H = prob["H"].cpu()
    E = prob["E"].cpu()
    ro = prob["row_offsets"].cpu()
    ids = prob["item_ids"].cpu()
    m = prob["row_mask"].cpu()
    V, D = E.shape
    valid = np.flatnonzero(m.numpy())
    rng = np.random.default_rng(0)
    n_items = 64
    items = rng.choice(V, size=n_items, replace=False)
    # calibrate on one row per thread, then size the sample to about target_s
    nt = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.rows(H, E, ro, ids, m, valid[:nt])
    t_batch = time.perf_counter() - t0
    n_rows = int(min(valid.size, max(nt, nt * math.floor(0.8 * target_s / max(t_batch, 1e-6)))))
    rows = rng.choice(valid, size=n_rows, replace=False)
    t0 = time.perf_counter()
    oracle.rows(H, E, ro, ids, m, rows)
    t_rows = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.items(H, E, ro, ids, m, items)
    t_items = time.perf_counter() - t0
    elems = n_rows * V + n_items * R_v          # (row, item) logits processed
    flops = 4.0 * D * elems                     # each side: logit dot + gradient axpy
    sec = t_rows + t_items
    return {
        "value": flops / sec / 1e12,
        "unit": "TFLOP/s",
        "rows_V_per_s": elems / 2.0 / sec,      # fwd+bwd elements: each (row, item) pair counted once per pass
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n_rows} valid rows x all {V} items (loss + dH) and {n_items} items x all {R_v} valid rows (dE), "
                  f"float64, {sec:.1f} s",
    }


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary; None when there is none or when the
    kernel sources changed after the counters were taken."""
    from vocabulary_label_bce_amd.profiling import source_digest

    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != source_digest():
        return None
    return d.get("bytes_per_launch")


def bench_topk(a, cfg, prob, R_v):
    """Full-vocabulary top-k scoring of every valid row of the workload (no [rows, V] buffer): 2*R_v*V*D flops."""
    import torch

    from vocabulary_label_bce_amd import binding as B
    from vocabulary_label_bce_amd.ops import topk

    H, E = prob["H"], prob["E"]
    ro, ids, m = prob["row_offsets"], prob["item_ids"], prob["row_mask"]
    V, D = E.shape
    ws = B.alloc_workspace(B.problem_of(H, E, ids), H.device)
    for _ in range(a.warmup):
        out = topk(H, E, a.topk, ro, ids, m, ws=ws)
    torch.cuda.synchronize()
    B.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        out = topk(H, E, a.topk, ro, ids, m, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = B.profile_read()
    B.profile_enable(False)
    ms = (t1 - t0) / a.steps * 1e3
    F = 2.0 * R_v * V * D
    tot, n = prof["topk_sweep"]
    sweep_ms = tot / n if n else None
    hits = out[2]
    valid = m.bool()
    print(json.dumps({
        "metric": f"full-vocabulary top-{a.topk} scoring TFLOP/s (rows.V/s)",
        "value": round(F / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "rows": cfg.R, "valid_rows": R_v, "D": D, "V": V, "k": a.topk},
        "rows_V_per_s": R_v * V / (ms * 1e-3),
        "kernels": {"topk_sweep": {"avg_ms": round(sweep_ms, 4) if sweep_ms else None, "launches": n,
                                   "tflops": round(F / (sweep_ms * 1e-3) / 1e12, 2) if sweep_ms else None}},
        "hit_at_k_all_valid_rows": float((hits[valid] > 0).float().mean().item()),
    }))


def mfma_ceiling(torch, B, dev, random_operands=False):
    """MFMA-only ceiling (cutbce_mfma_ceiling): one workgroup of 8 waves per CU (two per SIMD, as in the D = 128
    sweeps), each issuing v_mfma_f32_32x32x16_bf16 back to back from registers. Returns its rate and the shader
    clock the device held meanwhile (s_memtime over s_memrealtime ticks, median over waves). With
    random_operands (cutbce_mfma_ceiling_random) the operands are random bf16 values, as the sweeps' tiles are,
    so the clock includes the multipliers' data-dependent power."""
    run = B.mfma_ceiling_random if random_operands else B.mfma_ceiling
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    waves, iters = 8, 50000
    stamps = torch.zeros(4 * blocks * waves, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    run(blocks, waves, iters, stamps, stream)  # warm-up launch
    ev0.record(stream)
    run(blocks, waves, iters, stamps, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    st = stamps.view(-1, 4).double()
    ghz = (0.1 * (st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2])).median().item()
    tflops = blocks * waves * iters * 4 * 32768 / (ms * 1e-3) / 1e12
    name = "k_mfma_ceiling_random (random operands" if random_operands else \
        "k_mfma_ceiling (constant operands"
    return {"kernel": name + "; v_mfma_f32_32x32x16_bf16 from registers, 8 waves per CU)",
            "tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "clock_ghz": round(ghz, 3), "ms": round(ms, 3), "iters": iters, "blocks": blocks, "waves": waves}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": f"bench.py measures one GPU only (--gpus {a.gpus} requested): the library "
                                   "drives one GPU per process and has no multi-GPU mode"}))
        sys.exit(2)
    import torch

    from vocabulary_label_bce_amd import binding as B
    from vocabulary_label_bce_amd import workloads as W
    from vocabulary_label_bce_amd.ops import Workspace

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    B.lib()  # fail loudly before any work if the HIP library is missing
    cfg = W.CONFIGS[a.workload]
    dev = torch.device("cuda:0")
    prob = W.make_problem(cfg, seed=a.seed, device=dev)
    H, E = prob["H"], prob["E"]
    ro, ids, m = prob["row_offsets"], prob["item_ids"], prob["row_mask"]
    R_v = int(m.sum().item())
    V, D = E.shape
    if a.topk:
        return bench_topk(a, cfg, prob, R_v)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    mem_base, free0 = torch.cuda.memory_allocated(dev), torch.cuda.mem_get_info(dev)[0]
    w = Workspace(H, E, ids, want_row_loss=False, save_dh=True, want_metrics=a.metrics)
    g = torch.ones(1, dtype=torch.float32, device=dev)

    def step():
        w.forward(H, E, ro, ids, m)
        w.backward(H, E, ro, ids, m, grad=g, reuse=True)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    loss0 = float(w.loss.item())
    # device memory of the calls: the caching allocator's peak and the drop of free memory since before the
    # workspace and outputs were allocated, against a dense [rows, V] float32 logits buffer
    memory = {"workspace_bytes": w.ws.numel() * w.ws.element_size(),
              "allocator_peak_bytes": torch.cuda.max_memory_allocated(dev) - mem_base,
              "device_free_drop_bytes": free0 - torch.cuda.mem_get_info(dev)[0],
              "dense_logits_fp32_bytes": W.dense_logits_bytes(cfg.R, V)}
    B.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = B.profile_read()
    B.profile_enable(False)
    ms = (t1 - t0) / a.steps * 1e3
    if not math.isfinite(loss0):
        print(json.dumps({"error": "non-finite loss"}))
        sys.exit(1)

    F = 8.0 * R_v * V * D
    tflops = F / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    kern = {}
    for k, (tot, n) in prof.items():
        if n:
            avg = tot / n
            kern[k] = {"avg_ms": avg, "launches": n, "tflops": 4.0 * R_v * V * D / (avg * 1e-3) / 1e12}
    dom = max(kern, key=lambda k: kern[k]["avg_ms"]) if kern else None
    roof = None
    if dom:
        ach = kern[dom]["tflops"]
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": load_traffic(dom, a.workload),
                "flops_per_launch": 4.0 * R_v * V * D, "avg_launch_ms": round(kern[dom]["avg_ms"], 4)}
    out = {
        "metric": "fused BCE fwd+bwd TFLOP/s & % bf16 MFMA peak at V=876k (rows·V/s)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "N": cfg.N, "rows": cfg.R, "valid_rows": R_v, "D": D, "V": V,
                   "nnz": int(ids.numel()), "global_batch": cfg.B, "seq_len": cfg.N, "cut_metrics": a.metrics},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "rows_V_per_s": R_v * V / (ms * 1e-3),
        "credited_flops_per_step": F,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                    for k, d in kern.items()},
        "roofline": roof,
        "loss": loss0,
        "memory": memory,
    }
    for key, rnd in (("mfma_ceiling", False), ("mfma_ceiling_random", True)):
        ceil = mfma_ceiling(torch, B, dev, random_operands=rnd)
        if dom:
            ceil["dominant_kernel_frac_of_ceiling"] = round(kern[dom]["tflops"] / ceil["tflops"], 4)
        out[key] = ceil
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(prob, R_v, a.cpu_seconds)
    if a.copy_mib > 0:
        n = a.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        out["copy_calibration"] = {"kernel": "torch.neg float32", "bytes_read": 4 * n, "bytes_written": 4 * n,
                                   "launches": 3}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
