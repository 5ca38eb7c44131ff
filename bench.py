#!/usr/bin/env python3
"""Benchmark of the sparse decode offload step on one MI355X.

A step is one decode step of every layer of the workload: per layer, the new
token's rows are appended (device -> pinned host pool + device indexer) and
one sko_decode_step runs score -> packed top-k -> merge/dedupe -> LRU ->
miss gather -> remap -> attention for all sequences and positions.  The
metric is layer-steps/s over K timed steps that follow W warm-up steps (the
first of which is the all-miss cold step).  All inputs (prefix history,
per-step token rows and queries) are generated from the seeded synthetic
recipe and are resident on the device / in the pinned pool before timing.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the library's stream around every stage launch inside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
PCIE5_X16_GBPS = 63.0         # PCIe 5.0 x16 per direction, theoretical
IDX_ROW, KV_ROW = 128, 1152


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measure_h2d_ceiling(torch, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Bulk pinned host -> device copy rate (GB/s) of a 1 GiB buffer."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
    del src, dst
    return best


def cpu_baseline(w, target_s: float) -> dict:
    """The oracle as it stands, single-threaded, on layer 0 of the workload,
    all sequences, for as many decode steps as fit in about target_s."""
    import oracle
    o = oracle.Oracle(1, w.batch, w.capacity, w.top_k, w.hot_slots, w.positions, w.heads, 1.0 / 24.0)
    for b in range(w.batch):
        n = w.seq_context(b)
        o.append(0, b, w.index_rows(0, b, 0, n), w.kv_rows(0, b, 0, n))
    qs = [w.index_queries(0, b) for b in range(w.batch)]
    steps, elapsed = 0, 0.0
    while elapsed < target_s and steps < w.steps:
        t = steps
        rows_i = [w.index_rows(0, b, w.seq_context(b) + t, 1) for b in range(w.batch)]
        rows_k = [w.kv_rows(0, b, w.seq_context(b) + t, 1) for b in range(w.batch)]
        qi = np.stack([qs[b][t] for b in range(w.batch)])
        qa = np.stack([w.attn_queries(0, b, t) for b in range(w.batch)])
        t0 = time.perf_counter()
        for b in range(w.batch):
            o.append(0, b, rows_i[b], rows_k[b])
        o.decode_step(0, qi, qa)
        elapsed += time.perf_counter() - t0
        steps += 1
    o.close()
    return {"value": steps / elapsed, "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of '{w.name}', all {w.batch} sequences, decode steps 0..{steps - 1} "
                      f"(cold step included), {elapsed:.1f} s single-threaded"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=56)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="small")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-timing", action="store_true", help="time without per-stage events")
    ap.add_argument("--pool", choices=["default", "coherent", "noncoherent"], default="default",
                    help="host-pool allocation mode")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the offload step is "
              "per-GPU and this build has no multi-GPU path", file=sys.stderr)
        return 2

    import torch
    import synth
    import sparse_kv_offload_amd as sko

    w = synth.WORKLOADS[args.workload]
    L = args.layers or w.layers
    T = args.warmup + args.steps
    if T > w.steps:
        w = w.replace(steps=T)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    B, D, H, k = w.batch, w.positions, w.heads, w.top_k

    t_setup = time.perf_counter()
    flags = {"default": 0, "coherent": sko.SKO_FLAG_POOL_COHERENT,
             "noncoherent": sko.SKO_FLAG_POOL_NONCOHERENT}[args.pool]
    cfg = sko.make_config(num_layers=L, batch=B, max_tokens=w.capacity, num_heads=H, top_k=k,
                          hot_slots=w.hot_slots, mtp_positions=D, flags=flags)
    h = sko.SparseKVOffload(cfg, stream)
    chunk = 65536
    for l in range(L):
        for b in range(B):
            n = w.seq_context(b)
            for r0 in range(0, n, chunk):
                m = min(chunk, n - r0)
                h.append(l, b, w.index_rows(l, b, r0, m), w.kv_rows(l, b, r0, m))
    log(f"prefix loaded: {L}x{B}x{w.context} tokens in {time.perf_counter() - t_setup:.1f}s")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")

    # per-step inputs, resident on the device before timing
    new_idx, new_kv, q_idx, q_attn = [], [], [], []
    qchains = {(l, b): w.index_queries(l, b, T) for l in range(L) for b in range(B)}
    for t in range(T):
        new_idx.append([dev(np.concatenate([w.index_rows(l, b, w.seq_context(b) + t, 1) for b in range(B)]))
                        for l in range(L)])
        new_kv.append([dev(np.concatenate([w.kv_rows(l, b, w.seq_context(b) + t, 1) for b in range(B)]))
                       for l in range(L)])
        q_idx.append([dev(np.stack([qchains[(l, b)][t] for b in range(B)])) for l in range(L)])
        q_attn.append([dev(np.stack([w.attn_queries(l, b, t) for b in range(B)])) for l in range(L)])
    out = torch.empty((B, D, H, synth.V_DIM), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f}s")

    def run_step(t):
        for l in range(L):
            sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, new_idx[t][l], new_kv[t][l], 1, True)
            sko.sko_decode_step(h.handle, l, q_idx[t][l], q_attn[t][l], out)

    for t in range(args.warmup):
        run_step(t)
    torch.cuda.synchronize()
    stats0 = [h.stats(l) for l in range(L)]
    lt0 = w.context + args.warmup  # tokens present at the first timed step (after its append)

    h.set_timing(not args.no_timing)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, T):
        run_step(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timing = h.timing() if not args.no_timing else {}
    h.set_timing(False)
    stats1 = [h.stats(l) for l in range(L)]

    K = args.steps
    layer_steps = L * K
    value = layer_steps / elapsed
    d = {f: sum(getattr(s1, f) - getattr(s0, f) for s0, s1 in zip(stats0, stats1))
         for f in ("unique", "hits", "misses", "evictions", "h2d_bytes")}
    # algorithmic bytes per launch (averaged over the timed launches)
    avg_lt = lt0 + (K - 1) / 2.0
    scan_bytes = IDX_ROW * B * avg_lt + IDX_ROW * B * D
    gather_bytes = d["h2d_bytes"] / layer_steps
    attn_bytes = KV_ROW * B * D * min(k, avg_lt)

    h2d_ceiling = measure_h2d_ceiling(torch)

    rooflines = {}
    if timing:
        def kernel_avg_ms(name):
            ms, n = timing.get(name, (0.0, 0))
            return ms / n if n else float("nan")
        for name, nbytes, bound, peak in (
                ("score_hist", scan_bytes, "hbm", HBM_PEAK_GBPS),
                ("gather_misses", gather_bytes, "host-link", h2d_ceiling),
                ("attn_partial", attn_bytes, "hbm", HBM_PEAK_GBPS)):
            avg = kernel_avg_ms(name)
            ach = nbytes / (avg * 1e-3) / 1e9 if avg > 0 else 0.0
            rooflines[name] = {"bound": bound, "achieved": round(ach, 2), "peak": round(peak, 2),
                               "unit": "GB/s", "frac": round(ach / peak, 4), "traffic": None,
                               "avg_ms": round(avg, 5), "bytes_per_launch": int(nbytes)}
        dominant = max(timing.items(), key=lambda kv: kv[1][0])[0]
        roof = rooflines.get(dominant)
        if roof is None:  # a kernel without a bandwidth model dominates
            roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": None, "traffic": None}
        roof = dict(roof, kernel=dominant)
    else:
        roof, dominant = None, None

    result = {
        "metric": "sparse-offload decode layer-steps/s",
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "batch": B, "context": w.context,
                   "top_k": k, "hot_slots": w.hot_slots, "mtp_positions": D, "heads": H,
                   "parallelism": "none (1 GPU)", "pool": args.pool},
        "tokens_per_s": round(B * K / elapsed, 2),
        "indexer_scan_GBps": rooflines.get("score_hist", {}).get("achieved"),
        "miss_gather_GBps": rooflines.get("gather_misses", {}).get("achieved"),
        "h2d_ceiling_GBps": round(h2d_ceiling, 2),
        "hit_rate": round(d["hits"] / max(1, d["unique"]), 4),
        "unique_misses_per_layer_step": round(d["misses"] / layer_steps, 1),
        "h2d_bytes_per_layer_step": int(d["h2d_bytes"] / layer_steps),
        "roofline": roof,
        "rooflines": rooflines,
        "stage_ms_per_launch": {n: round(ms / c, 5) for n, (ms, c) in timing.items() if c},
    }
    h.close()
    del new_idx, new_kv, q_idx, q_attn
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
