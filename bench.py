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

Prints one JSON line.  Per-kernel durations come from HIP events that the
library records on its own stream: around every stage during the warm-up
steps after the cold one (the per-stage breakdown), and around the dominant
stage only during the timed steps (its roofline), since every event pair
costs device time.
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
HOST_LINK_PEAK_GBPS = 64.0    # MI355X host interface, PCIe 5.0 x16: 128 GB/s both ways
CALIB_COPY_BYTES = 256 << 20  # plain device copy run once for counter calibration
IDX_ROW, KV_ROW = 128, 1152
IDX_ROW_C8 = 64 + 2  # int8 codes + fp16 scale per token


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


def measure_hbm_copy(torch, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Device-to-device copy rate (GB/s, bytes read + written) of a 1 GiB
    buffer: a measured HBM ceiling beside the 8 TB/s vendor peak."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        dst.copy_(src)
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (time.perf_counter() - t0) / 1e9)
    del src, dst
    return best


def calibration_copy(torch) -> None:
    """One plain device-to-device copy of CALIB_COPY_BYTES, so that a counter
    run of this script also holds a kernel with known bytes read and written
    (the scale factor between the FETCH_SIZE / WRITE_SIZE counters and bytes)."""
    src = torch.ones(CALIB_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# Kernel source file that each modelled stage is compiled from.
KERNEL_SOURCE = {"score_hist": "select.hip", "gather_misses": "gather.hip", "merge_lru": "merge_lru.hip",
                 "attn_partial": "attention.hip"}


def code_digest(kernel_file: str) -> str:
    """Digest of a kernel's source file and of the runtime (which sets its
    launch shape), with comments and whitespace removed: only code changes
    alter it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in (kernel_file, "runtime.hip"):
        src = open(os.path.join(ROOT, "sparse_kv_offload_amd", "csrc", f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this kernel
    and workload, or None when there is none or the code of the kernel's
    source or of the runtime changed since the counters were taken (the
    summary records code_digest of both)."""
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    src = KERNEL_SOURCE.get(kernel)
    if not src or not os.path.isfile(path):
        return None
    m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
    if not m:
        return None
    entry = json.loads(m.group(1)).get(kernel)
    if not entry or entry.get("source_sha256_16") != code_digest(src):
        return None
    return entry.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """The host's CPU: logical CPUs, the CPUs this process may run on, and
    the model name the kernel reports."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


def _oracle_chains(w, seqs, nsteps, time_limit, barrier, results):
    """Worker of the CPU baseline: the oracle as it stands on layer 0 of the
    workload for the sequences `seqs` (chains are independent per (layer,
    sequence)), decode steps 0, 1, ... until nsteps are done or time_limit
    seconds have been spent in them.  Each step's inputs are generated before
    its timed region; only append + decode_step are timed.  Returns (steps,
    seconds inside the timed regions, wall clock at the start, at the end)."""
    import oracle
    o = oracle.Oracle(1, len(seqs), w.capacity, w.top_k, w.hot_slots, w.positions, w.heads, 1.0 / 24.0)
    for j, b in enumerate(seqs):
        n = w.seq_context(b)
        o.append(0, j, w.index_rows(0, b, 0, n), w.kv_rows(0, b, 0, n))
    qs = [w.index_queries(0, b, nsteps) for b in seqs]

    def inputs(t):
        return ([w.index_rows(0, b, w.seq_context(b) + t, 1) for b in seqs],
                [w.kv_rows(0, b, w.seq_context(b) + t, 1) for b in seqs],
                np.stack([q[t] for q in qs]),
                np.stack([w.attn_queries(0, b, t) for b in seqs]))

    # a worker of the all-core run holds every step's inputs before the
    # common start, so its wall time is oracle work only
    ready = [inputs(t) for t in range(nsteps)] if barrier is not None else [inputs(0)]
    if barrier is not None:
        barrier.wait()
    wall0, busy, t = time.time(), 0.0, 0
    while t < nsteps and busy < time_limit:
        rows_i, rows_k, qi, qa = ready[t] if barrier is not None else ready[0]
        t0 = time.perf_counter()
        for j in range(len(seqs)):
            o.append(0, j, rows_i[j], rows_k[j])
        o.decode_step(0, qi, qa)
        busy += time.perf_counter() - t0
        t += 1
        if barrier is None and t < nsteps:
            ready[0] = inputs(t)
    wall1 = time.time()
    o.close()
    if results is not None:
        results.put((t, busy, wall0, wall1))
    return t, busy, wall0, wall1


def cpu_baseline(w, target_s: float, max_workers: int = 16) -> dict:
    """The oracle as it stands, timed on the host cores on layer 0 of the
    workload, all sequences, decode steps from the cold step on.  First on one
    thread, for about target_s; then with the independent sequence chains
    spread over worker processes (one oracle per worker, sequences dealt
    round-robin) on every CPU this process may use, at most max_workers, for
    about target_s of wall time.  The oracle's arithmetic is the same in both;
    the all-core rate is the step count over the wall time from the common
    start to the last worker's end."""
    import multiprocessing as mp
    host = host_cpu()
    n1, busy, _, _ = _oracle_chains(w, list(range(w.batch)), w.steps, target_s, None, None)
    single = {"value": round(n1 / busy, 4), "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
              "sample": f"layer 0 of '{w.name}', all {w.batch} sequences, decode steps 0..{n1 - 1} "
                        f"(cold step included), {busy:.1f} s on one thread"}
    workers = max(1, min(w.batch, host["affinity"], max_workers))
    per_worker = -(-w.batch // workers)
    # steps that fill about target_s on the slowest worker (it holds per_worker chains)
    nsteps = max(1, min(w.steps, int(target_s * n1 / busy * w.batch / per_worker)))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_chains,
                         args=(w, list(range(j, w.batch, workers)), nsteps, float("inf"), barrier, results))
             for j in range(workers)]
    # one thread per worker: the input generator's own OpenMP pool would
    # otherwise oversubscribe the cores the workers share
    omp = os.environ.get("OMP_NUM_THREADS")
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        for pr in procs:
            pr.start()
    finally:
        if omp is None:
            del os.environ["OMP_NUM_THREADS"]
        else:
            os.environ["OMP_NUM_THREADS"] = omp
    got = [results.get() for _ in procs]
    for pr in procs:
        pr.join()
    if any(pr.exitcode != 0 for pr in procs):
        raise RuntimeError("an oracle worker failed")
    wall = max(g[3] for g in got) - min(g[2] for g in got)
    return {"value": round(nsteps / wall, 4), "unit": "layer-steps/s", "cores": workers, "kind": "oracle",
            "sample": f"layer 0 of '{w.name}', all {w.batch} sequences dealt over {workers} worker processes "
                      f"(one oracle each), decode steps 0..{nsteps - 1} (cold step included), "
                      f"{wall:.1f} s wall",
            "single_thread": single, "host": host}


class _DeviceBytes:
    """A device address seen by torch as a uint8 tensor (no copy)."""

    def __init__(self, ptr: int, nbytes: int):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False),
                                         "version": 3, "strides": None, "stream": None}


def prefill_bench(args) -> int:
    """Layerwise prefill offload: N layers, B0 bound to layer 0, three
    rotating trays; each pass loads every layer's cached prefix (host ->
    device), runs a stand-in for the layer's compute of a chosen duration on
    the compute stream (a timed spin kernel), writes the chunk's new rows and
    saves them (device -> host).  Reports the measured exposed delay per
    layer next to the model max(0, load - compute of the previous layer)."""
    import torch
    import sparse_kv_offload_amd as sko
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    N, row, prefix, chunk = args.prefill_layers, 1152, args.prefill_prefix, args.prefill_chunk
    passes = 2
    cap = prefix + passes * chunk
    # calibrate the spin kernel: cycles per millisecond
    torch.cuda._sleep(1000000)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(50000000)
    torch.cuda.synchronize()
    cyc_per_ms = 50000000 / ((time.perf_counter() - t0) * 1e3)
    rows = torch.randint(0, 256, (chunk * row,), dtype=torch.uint8, device="cuda")
    results = []
    with sko.PrefillOffload(N, 3, 1, row, cap, independent=[1] + [0] * (N - 1), stream=stream) as pf:
        rng = np.random.default_rng(5)
        pat = rng.integers(0, 256, size=(min(prefix, 4096), row), dtype=np.uint8)
        for l in range(N):
            hp = pf.host_pool(l)
            for r0 in range(0, prefix, pat.shape[0]):
                m = min(pat.shape[0], prefix - r0)
                hp[r0:r0 + m] = pat[:m]
            pf.set_tokens(l, prefix)
        load_ms_est = prefix * row / 55e9 * 1e3
        for frac in args.prefill_compute:
            comp_ms = frac * load_ms_est
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for l in range(N):
                ptr = pf.begin_layer(l)
                if comp_ms > 0:
                    torch.cuda._sleep(int(comp_ms * cyc_per_ms))
                P_l = pf.tokens(l)
                buf = torch.as_tensor(_DeviceBytes(ptr, cap * row), device="cuda")
                buf[P_l * row:(P_l + chunk) * row].copy_(rows)
                # the alias of the library's buffer ends with the layer
                del buf
                pf.end_layer(l, chunk)
            pf.sync()
            wall = time.perf_counter() - t0
            t = [pf.layer_timing(l) for l in range(N)]
            load = [x[0] for x in t]
            exp = [x[1] for x in t]
            comp = [x[2] for x in t]
            model = [max(0.0, load[l] - comp[l - 1]) if l > 0 else load[0] for l in range(N)]
            results.append({"compute_ms_per_layer": round(float(np.mean(comp[1:])), 3),
                            "load_ms_per_layer": round(float(np.mean(load[1:])), 3),
                            "load_GBps": round(prefix * row / (np.mean(load[1:]) * 1e-3) / 1e9, 2),
                            "exposed_ms_sum": round(float(sum(exp[1:])), 3),
                            "model_exposed_ms_sum": round(float(sum(model[1:])), 3),
                            "pass_ms": round(wall * 1e3, 2),
                            "pass_ms_if_resident": round(float(sum(comp)), 2)})
            # the next setting starts from the same prefix
            for l in range(N):
                pf.set_tokens(l, prefix)
        # nothing queued on any stream may touch the library's buffers once
        # the handle is destroyed
        torch.cuda.synchronize()
        pf.sync()
    del rows
    torch.cuda.synchronize()
    print(json.dumps({"metric": "layerwise prefill offload: exposed transfer delay per pass",
                      "unit": "ms", "layers": N, "row_bytes": row, "prefix_tokens": prefix,
                      "chunk_tokens": chunk, "trays": "B0 bound to layer 0 + 3 rotating", "lookahead": 1,
                      "tray_footprint_ratio": round(4 / N, 4), "settings": results}), flush=True)
    return 0


def cache_management(calib, overlap):
    """Selection (score pass, filter, refine) plus the LRU update of one
    layer-step, in µs, from the event-timed warm-up stages.  With the late or
    fused copy the LRU-update launch does no copy and its stage time is the
    update itself; with the early copy the launch also holds the copy blocks,
    and the update is the span of its merge blocks (block stamps), which run
    beside the copy."""
    if not calib:
        return None
    per = {n: ms / c * 1e3 for n, (ms, c) in calib.items() if c}
    sel = sum(per.get(n, 0.0) for n in ("score_hist", "topk_filter", "topk_refine"))
    if overlap is None or not overlap["launches"] or overlap["copy_ms"] <= 0:
        lru, src = per.get("merge_lru", 0.0), "merge_lru stage (no copy blocks in the launch)"
    else:
        lru, src = overlap["merge_ms"] / overlap["launches"] * 1e3, "merge blocks' span beside the copy blocks"
    return {"selection_us": round(sel, 2), "lru_update_us": round(lru, 2), "total_us": round(sel + lru, 2),
            "lru_update_source": src}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=56)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="shelf_ctx8",
                    help="tiny, small, mtp3, shelf_ctx8 (the largest single-GPU workload; default), "
                         "shelf_ctx4 or long")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="about this long for each of the two oracle timings (one thread, all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-timing", action="store_true", help="time without per-stage events")
    ap.add_argument("--indexer", choices=["bf16", "c8"], default="bf16",
                    help="indexer cache: bf16 rows, or int8 codes with fp16 scales after a Hadamard rotation")
    ap.add_argument("--pool", choices=["default", "coherent", "noncoherent"], default="default",
                    help="host-pool allocation mode")
    ap.add_argument("--append", choices=["fused", "separate"], default="fused",
                    help="append each step's token inside the decode call (sko_decode_step_append) or with "
                         "its own call (sko_append_token, then sko_decode_step)")
    ap.add_argument("--copy", choices=["default", "early", "late", "fused"], default="default",
                    help="miss-copy arrangement: early (the default: by extra blocks of the LRU-update launch), "
                         "late (after the LRU update), fused (inside the attention launch; one "
                         "position, at most 16 heads)")
    ap.add_argument("--micro-batches", type=int, default=0,
                    help="split the batch into this many handles on as many streams, kept off the copy XCD "
                         "(0: two when the batch has at least 2 sequences, else one)")
    ap.add_argument("--xcd-split", action="store_true",
                    help="keep the step's kernels off the copy blocks' XCD even with one micro-batch")
    ap.add_argument("--hit-overlap", action="store_true",
                    help="with the early copy: attend the resident rows on a side stream beside the copy launch, "
                         "the missed rows after it")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the layerwise prefill offload pipeline instead of the decode step")
    ap.add_argument("--prefill-layers", type=int, default=78)
    ap.add_argument("--prefill-prefix", type=int, default=32768)
    ap.add_argument("--prefill-chunk", type=int, default=4096)
    ap.add_argument("--prefill-compute", type=float, nargs="+", default=[0.0, 0.5, 1.0, 2.0],
                    help="compute per layer as multiples of the estimated load time")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the offload step is "
              "per-GPU and this library has no multi-GPU path", file=sys.stderr)
        return 2
    if args.prefill:
        return prefill_bench(args)

    import synth

    w = synth.WORKLOADS[args.workload]
    L = args.layers or w.layers
    T = args.warmup + args.steps
    if T > w.steps:
        w = w.replace(steps=T)
    # The oracle's timing runs first, in worker processes started before this
    # process touches the GPU.
    cpu_base = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        cpu_base = cpu_baseline(w, args.cpu_baseline_seconds)
        log(f"oracle: {cpu_base['single_thread']['value']} layer-steps/s on 1 thread, "
            f"{cpu_base['value']} on {cpu_base['cores']}")

    import torch
    import sparse_kv_offload_amd as sko
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    B, D, H, k = w.batch, w.positions, w.heads, w.top_k

    t_setup = time.perf_counter()
    flags = {"default": 0, "coherent": sko.SKO_FLAG_POOL_COHERENT,
             "noncoherent": sko.SKO_FLAG_POOL_NONCOHERENT}[args.pool]
    flags |= {"default": 0, "early": sko.SKO_FLAG_EARLY_COPY, "late": sko.SKO_FLAG_LATE_COPY,
              "fused": sko.SKO_FLAG_FUSED_COPY}[args.copy]
    if args.indexer == "c8":
        flags |= sko.SKO_FLAG_INDEXER_C8
    if args.hit_overlap:
        flags |= sko.SKO_FLAG_HIT_OVERLAP
    # Micro-batches: the batch is split into NMB contiguous groups of
    # sequences, one handle and one stream each, every handle kept off the
    # XCD of the copy blocks, so that one group's selection and attention run
    # while another group's misses cross the host link.  Each layer-step
    # issues every group's call for the layer before the next layer's.
    # two micro-batches wherever the batch has two sequences or more
    # (measured, one box each, layer-steps/s, one handle -> two: shelf_ctx8
    # 2 743 -> 3 402, mtp3 1 239 -> 1 403, small 5 007 -> 5 371, long
    # 4 363 -> 4 767)
    nmb = args.micro_batches if args.micro_batches > 0 else (2 if B >= 2 else 1)
    nmb = max(1, min(nmb, B))
    if nmb > 1 or args.xcd_split:
        flags |= sko.SKO_FLAG_XCD_SPLIT
    groups = [list(range(g * B // nmb, (g + 1) * B // nmb)) for g in range(nmb)]
    streams = [stream] if nmb == 1 else [torch.cuda.Stream() for _ in range(nmb)]
    hs = []
    split_note = None
    for g, seqs in enumerate(groups):
        cfg = sko.make_config(num_layers=L, batch=len(seqs), max_tokens=w.capacity, num_heads=H, top_k=k,
                              hot_slots=w.hot_slots, mtp_positions=D, flags=flags)
        try:
            hs.append(sko.SparseKVOffload(cfg, streams[g]))
        except sko.SkoError as e:
            if not (flags & sko.SKO_FLAG_XCD_SPLIT) or e.code != sko.SKO_E_UNSUPPORTED or hs:
                raise
            # a device that does not deal launch blocks in the fixed stripe:
            # one handle over the whole batch, without the split
            split_note = f"XCD split unsupported on this device ({e}); one handle"
            log(split_note)
            flags &= ~sko.SKO_FLAG_XCD_SPLIT
            nmb, groups, streams = 1, [list(range(B))], [stream]
            cfg = sko.make_config(num_layers=L, batch=B, max_tokens=w.capacity, num_heads=H, top_k=k,
                                  hot_slots=w.hot_slots, mtp_positions=D, flags=flags)
            hs.append(sko.SparseKVOffload(cfg, stream))
            break
    chunk = 65536
    for h, seqs in zip(hs, groups):
        for l in range(L):
            for j, b in enumerate(seqs):
                n = w.seq_context(b)
                for r0 in range(0, n, chunk):
                    m = min(chunk, n - r0)
                    h.append(l, j, w.index_rows(l, b, r0, m), w.kv_rows(l, b, r0, m))
    torch.cuda.synchronize()
    log(f"prefix loaded: {L}x{B}x{w.context} tokens in {time.perf_counter() - t_setup:.1f}s")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")

    # per-step inputs, resident on the device before timing
    new_idx, new_kv, q_idx, q_attn = [], [], [], []
    qchains = {(l, b): w.index_queries(l, b, T) for l in range(L) for b in range(B)}
    # [t][l][group]
    for t in range(T):
        new_idx.append([[dev(np.concatenate([w.index_rows(l, b, w.seq_context(b) + t, 1) for b in seqs]))
                         for seqs in groups] for l in range(L)])
        new_kv.append([[dev(np.concatenate([w.kv_rows(l, b, w.seq_context(b) + t, 1) for b in seqs]))
                        for seqs in groups] for l in range(L)])
        q_idx.append([[dev(np.stack([qchains[(l, b)][t] for b in seqs])) for seqs in groups] for l in range(L)])
        q_attn.append([[dev(np.stack([w.attn_queries(l, b, t) for b in seqs])) for seqs in groups]
                       for l in range(L)])
    outs = [torch.empty((len(seqs), D, H, synth.V_DIM), dtype=torch.float32, device="cuda") for seqs in groups]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f}s")

    def run_step(t):
        for l in range(L):
            for g, h in enumerate(hs):
                if args.append == "fused":
                    # the new token's rows go in with the decode call (one
                    # launch fewer per layer-step; same results as the two calls)
                    sko.sko_decode_step_append(h.handle, l, new_idx[t][l][g], new_kv[t][l][g], q_idx[t][l][g],
                                               q_attn[t][l][g], outs[g])
                else:
                    sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, new_idx[t][l][g], new_kv[t][l][g], 1, True)
                    sko.sko_decode_step(h.handle, l, q_idx[t][l][g], q_attn[t][l][g], outs[g])

    def all_stats():
        # per (group, layer); the counters are summed over both
        return [h.stats(l) for h in hs for l in range(L)]

    def set_timing(mask):
        for h in hs:
            h.set_timing(mask)

    def merged_timing():
        m = {}
        for h in hs:
            for name, (ms, c) in h.timing().items():
                a = m.get(name, (0.0, 0))
                m[name] = (a[0] + ms, a[1] + c)
        return m

    def merged_overlap():
        m = None
        for h in hs:
            o = h.copy_overlap()
            m = dict(o) if m is None else {key: m[key] + o[key] for key in m}
        return m

    # Warm-up: the cold step untimed, then the remaining warm-up steps with
    # every stage bracketed by events (the per-stage breakdown; each event
    # pair costs device time, so the timed steps bracket only one stage).
    nstage = sko.sko_num_stages()
    stats_cold0 = all_stats()
    torch.cuda.synchronize()
    t_cold = time.perf_counter()
    run_step(0)
    torch.cuda.synchronize()
    t_cold = time.perf_counter() - t_cold
    calib_stats0 = all_stats()
    set_timing(0 if args.no_timing else (1 << nstage) - 1)
    for t in range(1, args.warmup):
        run_step(t)
    torch.cuda.synchronize()
    calib = merged_timing() if (not args.no_timing and args.warmup > 1) else {}
    stats0 = all_stats()
    calib_steps = args.warmup - 1

    dominant = None
    if calib:
        dominant = max(calib.items(), key=lambda kv: kv[1][0])[0]
    timed_mask = 0 if dominant is None else (1 << sko.sko_stage_index(dominant))
    set_timing(timed_mask)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, T):
        run_step(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timing = merged_timing() if timed_mask else {}
    # block stamps of the timed LRU-update launches (early copy): how long the
    # copy blocks ran beside the LRU update
    overlap = merged_overlap() if timed_mask else None
    # the copy spans of every timed LRU-update launch of every handle, on the
    # device clock: their union is the time during which any missed row is
    # being copied over the host link
    span_list, span_khz = [], None
    if timed_mask and dominant == "merge_lru":
        for h in hs:
            sp, span_khz = h.copy_spans()
            span_list.append(sp)
    set_timing(0)
    stats1 = all_stats()

    K = args.steps
    layer_steps = L * K
    value = layer_steps / elapsed

    def union_s(spans_per_handle, khz):
        """Total length (s) of the union of [start, end) spans in ticks."""
        iv = sorted((int(a), int(b)) for sp in spans_per_handle for a, b in sp if b > a)
        tot, cur = 0, None
        for a, b in iv:
            if cur is None or a > cur[1]:
                if cur:
                    tot += cur[1] - cur[0]
                cur = [a, b]
            else:
                cur[1] = max(cur[1], b)
        if cur:
            tot += cur[1] - cur[0]
        return tot / (khz * 1e3)

    def deltas(s0, s1):
        return {f: sum(getattr(b, f) - getattr(a, f) for a, b in zip(s0, s1))
                for f in ("unique", "hits", "misses", "evictions", "h2d_bytes", "rescans", "direct_rows")}

    d = deltas(stats0, stats1)

    def alg_bytes(first_step, nsteps, h2d_bytes, mode):
        """Algorithmic bytes per launch of the modelled kernels, averaged over
        decode steps first_step .. first_step + nsteps - 1.  The launch that
        reads the missed rows over the host link is bound by it: the
        attention (mode "fused"), the copy blocks of the merge launch
        ("early") or the gather ("late"); each missed row is written once,
        into the row its slot takes over, and the attention reads the
        winners' rows."""
        avg_lt = w.context + first_step + (nsteps + 1) / 2.0  # tokens present after each append
        ls = L * nsteps * nmb  # launches of each kernel (one per group and layer-step)
        per = h2d_bytes / ls if ls else 0.0
        Bg = B / nmb  # sequences per launch
        copy = (per, "host-link", HOST_LINK_PEAK_GBPS)
        # the query rows are read as bf16 in both modes
        idx_row = IDX_ROW_C8 if args.indexer == "c8" else IDX_ROW
        m = {"score_hist": (idx_row * Bg * avg_lt + IDX_ROW * Bg * D, "hbm", HBM_PEAK_GBPS)}
        if mode == "fused":
            m["attn_partial"] = copy
            return m
        attn = KV_ROW * Bg * D * min(k, avg_lt)
        if mode == "early":
            m["merge_lru"] = copy  # its copy blocks read the missed rows from the host
        else:
            m["gather_misses"] = copy
        m["attn_partial"] = (attn, "hbm", HBM_PEAK_GBPS)
        return m

    def copy_mode(t):
        return {"late": "late", "fused": "fused"}.get(args.copy, "early")

    h2d_ceiling = measure_h2d_ceiling(torch)
    zero_copy = sko.sko_link_read_rate(0, 1 << 30, 3)
    # the attention's access pattern (random whole rows, cold) at this
    # workload's shape, B*D lists of k rows, each list over its own region
    # of up to 4k rows: the practical HBM ceiling of the attention
    gather_rows = min(k, w.context) // 128 * 128
    gather_slots = max(gather_rows, min(w.hot_slots, 4 * gather_rows))
    gather_ceiling = sko.sko_hbm_gather_rate(0, B * D, gather_slots, gather_rows, 2) \
        if gather_rows >= 128 and B * D * gather_slots <= (1 << 22) else None
    # a plain streaming read of 256 MiB (cold): the practical HBM ceiling of
    # the indexer score pass, which reads every indexer row once
    stream_ceiling = sko.sko_hbm_read_rate(0, 1 << 28, 5)
    hbm_copy = measure_hbm_copy(torch)
    calibration_copy(torch)

    # the counter summary of this configuration under profiles/
    profile_name = (w.name + ("_c8" if args.indexer == "c8" else "") + (f"_mb{nmb}" if nmb > 1 else "")
                    + ("_xcd" if nmb == 1 and args.xcd_split else ""))

    def roof_entry(name, ms, n, model):
        nbytes, bound, peak = model[name]
        avg = ms / n
        ach = nbytes / (avg * 1e-3) / 1e9 if avg > 0 else 0.0
        e = {"bound": bound, "achieved": round(ach, 2), "peak": round(peak, 2), "unit": "GB/s",
             "frac": round(ach / peak, 4), "traffic": traffic_for(name, profile_name), "kernel": name,
             "avg_ms": round(avg, 5), "launches": n, "bytes_per_launch": int(nbytes)}
        if bound == "host-link":
            e["measured_ceiling"] = round(h2d_ceiling, 2)
            e["frac_of_measured"] = round(ach / h2d_ceiling, 4)
        elif name == "attn_partial" and gather_ceiling:
            e["measured_ceiling"] = round(gather_ceiling, 1)
            e["frac_of_measured"] = round(ach / gather_ceiling, 4)
        elif name == "score_hist" and stream_ceiling:
            e["measured_ceiling"] = round(stream_ceiling, 1)
            e["frac_of_measured"] = round(ach / stream_ceiling, 4)
        return e

    rooflines = {}
    if calib:
        model = alg_bytes(1, calib_steps, deltas(calib_stats0, stats0)["h2d_bytes"], copy_mode(calib))
        for name in model:
            ms, n = calib.get(name, (0.0, 0))
            if n:
                rooflines[name] = roof_entry(name, ms, n, model)
    roof = None
    if timing and dominant in timing:
        model = alg_bytes(args.warmup, K, d["h2d_bytes"], copy_mode(calib))
        ms, n = timing[dominant]
        if dominant in model:
            roof = roof_entry(dominant, ms, n, model)
        else:  # a kernel without a byte model dominates: report its time only
            roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": None, "traffic": None, "kernel": dominant, "avg_ms": round(ms / n, 5)}

    copy_union_s = None
    if span_list and span_khz and sum(len(sp) for sp in span_list) == layer_steps * nmb:
        copy_union_s = union_s(span_list, span_khz) or None
    if roof is not None and roof.get("bound") == "host-link" and elapsed > 0:
        # with micro-batches the copy launches of the handles overlap and
        # share the link, so a launch's own rate is a share of it; the link's
        # rate over the timed steps is the copied bytes over the wall time
        roof["concurrent_handles"] = nmb
        roof["link_rate_over_timed_steps_GBps"] = round(d["h2d_bytes"] / elapsed / 1e9, 2)
        roof["link_rate_frac_of_measured"] = round(d["h2d_bytes"] / elapsed / 1e9 / h2d_ceiling, 4)
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
                   "parallelism": "none (1 GPU)", "pool": args.pool, "copy": args.copy,
                   "hit_overlap": bool(args.hit_overlap), "append": args.append,
                   "indexer": args.indexer, "micro_batches": nmb,
                   "xcd_split": bool(flags & sko.SKO_FLAG_XCD_SPLIT),
                   **({"note": split_note} if split_note else {})},
        "tokens_per_s": round(B * K / elapsed, 2),
        "indexer_scan_GBps": rooflines.get("score_hist", {}).get("achieved"),
        # the miss gather's host-link rate: copied bytes over the time during
        # which any copy block runs (the union of every handle's copy spans;
        # with one handle, the copy blocks' own time), when every timed launch
        # was recorded; else the per-launch rate of the roofline
        "miss_gather_GBps": (round(d["h2d_bytes"] / copy_union_s / 1e9, 2) if copy_union_s else
                             next((e["achieved"] for e in [roof or {}] + list(rooflines.values())
                                   if e.get("bound") == "host-link"), None)),
        "miss_gather": ({"GBps": round(d["h2d_bytes"] / copy_union_s / 1e9, 2),
                         "frac_of_measured": round(d["h2d_bytes"] / copy_union_s / 1e9 / h2d_ceiling, 4),
                         "copy_busy_us_per_layer_step": round(copy_union_s / layer_steps * 1e6, 2),
                         "copy_busy_frac_of_wall": round(copy_union_s / elapsed, 4),
                         "launches": int(sum(len(sp) for sp in span_list)),
                         "definition": "copied bytes / union of all handles' copy spans (first copy block start "
                                       "to last copy block end of each LRU-update launch, device clock)"}
                        if copy_union_s else None),
        "miss_copy": copy_mode(calib) if calib else None,
        "h2d_ceiling_GBps": round(h2d_ceiling, 2),
        # a streaming kernel reading contiguous pinned host memory
        "zero_copy_read_GBps": round(zero_copy, 2),
        # random whole-row gathers from HBM (the attention's access pattern)
        "hbm_row_gather_GBps": round(gather_ceiling, 1) if gather_ceiling else None,
        # a plain streaming read of HBM (the score pass's access pattern)
        "hbm_stream_read_GBps": round(stream_ceiling, 1),
        "hbm_copy_GBps": round(hbm_copy, 1),
        # the first step finds an empty shelf (every winner a miss); it is
        # not in `value`
        "cold_step": {"ms": round(t_cold * 1e3, 3), "layer_steps_per_s": round(L / t_cold, 1),
                      "h2d_bytes_per_layer_step": int(deltas(stats_cold0, calib_stats0)["h2d_bytes"] / L)},
        "hit_rate": round(d["hits"] / max(1, d["unique"]), 4),
        "unique_misses_per_layer_step": round(d["misses"] / layer_steps, 1),
        "h2d_bytes_per_layer_step": int(d["h2d_bytes"] / layer_steps),
        # the host link alone, at the measured bulk rate, would allow this
        # many layer-steps/s; value / link_bound = share of the layer-step
        # during which the link carries misses at that rate
        "link_bound_layer_steps_per_s": round(h2d_ceiling * 1e9 * layer_steps / d["h2d_bytes"], 1)
        if d["h2d_bytes"] else None,
        "frac_of_link_bound": round(value * d["h2d_bytes"] / (h2d_ceiling * 1e9 * layer_steps), 4)
        if d["h2d_bytes"] else None,
        # the miss transfer against the rest of the step: the copy span and the
        # LRU-update span of each timed copy launch and their intersection
        # (the share of the copy during which other step work runs), and the
        # part of a layer-step not covered by the link at its measured rate
        "copy_overlap": ({
            "launches": overlap["launches"],
            "copy_span_us": round(overlap["copy_ms"] / overlap["launches"] * 1e3, 2),
            "merge_span_us": round(overlap["merge_ms"] / overlap["launches"] * 1e3, 2),
            "overlapped_us": round(overlap["overlap_ms"] / overlap["launches"] * 1e3, 2),
            "overlap_frac_of_copy": round(overlap["overlap_ms"] / overlap["copy_ms"], 4),
            "link_time_us_per_layer_step": round(d["h2d_bytes"] / layer_steps / (h2d_ceiling * 1e9) * 1e6, 2),
            "exposed_non_link_us_per_layer_step": round(
                elapsed / layer_steps * 1e6 - d["h2d_bytes"] / layer_steps / (h2d_ceiling * 1e9) * 1e6, 2),
        } if overlap and overlap["launches"] and overlap["copy_ms"] > 0 else None),
        # the selection and LRU bookkeeping of a layer-step, the miss copy
        # excluded (the pages' "cache management" per indexer layer)
        "cache_management_us_per_layer_step": cache_management(calib, overlap),
        "selection_rescans": d["rescans"],
        "newest_rows_from_device": d["direct_rows"],
        "roofline": roof,
        "rooflines": rooflines,
        "stage_ms_per_launch": {n: round(ms / c, 5) for n, (ms, c) in calib.items() if c},
        "stage_timing_note": (f"stage breakdown from warm-up steps 1..{args.warmup - 1} with every stage "
                              f"event-timed" + (f", the {nmb} handles' steps overlapping as in the timed steps (a "
                                                f"stage's time includes waiting behind the other handle's kernels)"
                                                if nmb > 1 else "") +
                              f"; the timed steps bracket only '{dominant}'")
        if calib else None,
    }
    for h in hs:
        h.close()
    del new_idx, new_kv, q_idx, q_attn
    if cpu_base is not None:
        result["cpu_baseline"] = cpu_base
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
