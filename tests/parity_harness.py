"""Side-by-side runs of the HIP path (through the C ABI) and the CPU oracle.

Both sides consume the same seeded inputs from ``synth``; nothing computed by
one side is fed to the other.  ``compare_step`` states the parity bar:
  * bit-exact: packed winners (index + miss flag, compared as sets per
    position since the order of winners is free), their hot slots, per-seq
    counts, the miss list, victims and evicted owners (in victim order), and
    the full residency tables and hot-buffer bytes after the step (with the
    int8 indexer also its codes and fp16 scales);
  * attention: |gpu - oracle| <= 2e-2 absolute for every element, and a
    relative RMS error per (seq, position, head) of at most ATTN_REL_RMS.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth

ATTN_ABS_TOL = 2e-2
# bf16 rounding of the probabilities fed to the P.V product bounds the
# relative error near 2^-9 per term; 1e-2 leaves margin for fp32 sums.
ATTN_REL_RMS = 1e-2
SCALE = 1.0 / 24.0


def torch_mod():
    import torch
    return torch


def to_device_u16(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


@dataclasses.dataclass
class StepResult:
    topk: np.ndarray
    phys: np.ndarray
    counts: np.ndarray
    misses: np.ndarray
    victims: np.ndarray
    evict_old: np.ndarray
    out: Optional[np.ndarray]
    keys: Optional[np.ndarray] = None


class Inputs:
    """Per-(layer, seq) query streams of a workload, generated once."""

    def __init__(self, w: synth.Workload, layers: List[int], steps: int):
        self.w = w
        self.steps = steps
        self.q_idx = {(l, b): w.index_queries(l, b, steps) for l in layers for b in range(w.batch)}

    def q_idx_step(self, layer: int, t: int, seqs: List[int]) -> np.ndarray:
        return np.stack([self.q_idx[(layer, b)][t] for b in seqs])

    def q_attn_step(self, layer: int, t: int, seqs: List[int]) -> np.ndarray:
        return np.stack([self.w.attn_queries(layer, b, t) for b in seqs])


class GpuSide:
    """The HIP path through the C ABI: one handle over the workload's
    sequences `seqs` (all of them by default; the handle's sequence j is the
    workload's seqs[j]), on `stream` (the current one by default)."""

    def __init__(self, w: synth.Workload, layers: int, device_append: bool = True,
                 prefix_chunk: int = 65536, flags: int = 0, fused_append: bool = False,
                 seqs: Optional[List[int]] = None, stream=None):
        import sparse_kv_offload_amd as sko
        torch = torch_mod()
        self.sko, self.torch, self.w = sko, torch, w
        self.L = layers
        self.seqs = list(range(w.batch)) if seqs is None else list(seqs)
        cfg = sko.make_config(num_layers=layers, batch=len(self.seqs), max_tokens=w.capacity,
                              num_heads=w.heads, top_k=w.top_k, hot_slots=w.hot_slots,
                              mtp_positions=w.positions, attn_scale=SCALE, flags=flags)
        self.stream = torch.cuda.current_stream() if stream is None else stream
        self.h = sko.SparseKVOffload(cfg, self.stream)
        self.device_append = device_append
        self.prefix_chunk = prefix_chunk
        # fused_append: each step's token goes in with the decode call
        # (sko_decode_step_append) instead of sko_append_token
        self.fused_append = fused_append
        self.pending = {}
        self._keep = []

    def close(self):
        self.h.close()

    def load_prefix(self, layer: int, seq: int, n: Optional[int] = None) -> None:
        """Prefix of the handle's sequence `seq` (workload sequence seqs[seq])."""
        ws = self.seqs[seq]
        n = self.w.seq_context(ws) if n is None else n
        for r0 in range(0, n, self.prefix_chunk):
            m = min(self.prefix_chunk, n - r0)
            self.h.append(layer, seq, self.w.index_rows(layer, ws, r0, m), self.w.kv_rows(layer, ws, r0, m))

    def append_token(self, layer: int, t: int) -> None:
        w = self.w
        idx = np.concatenate([w.index_rows(layer, b, w.seq_context(b) + t, 1) for b in self.seqs])
        kv = np.concatenate([w.kv_rows(layer, b, w.seq_context(b) + t, 1) for b in self.seqs])
        if self.fused_append:
            self.pending[layer] = (to_device_u16(idx), to_device_u16(kv))
        elif self.device_append:
            di, dk = to_device_u16(idx), to_device_u16(kv)
            self.stream.wait_stream(self.torch.cuda.current_stream())
            self.h.append(layer, self.sko.SKO_ALL_SEQS, di, dk, 1)
            self._keep.append((di, dk))
        else:
            self.h.append(layer, self.sko.SKO_ALL_SEQS, idx, kv, 1)

    def issue(self, layer: int, q_idx: np.ndarray, q_attn: np.ndarray):
        """Queues the decode step of `layer` (queries of the handle's
        sequences) without waiting for it; returns its output tensor."""
        torch = self.torch
        w = self.w
        qi, qa = to_device_u16(q_idx), to_device_u16(q_attn)
        out = torch.empty((len(self.seqs), w.positions, w.heads, synth.V_DIM), dtype=torch.float32, device="cuda")
        # inputs made on the current stream are complete before the step
        self.stream.wait_stream(torch.cuda.current_stream())
        if layer in self.pending:
            idx, kv = self.pending.pop(layer)
            self.h.decode_step_append(layer, idx, kv, qi, qa, out)
            self._keep.append((idx, kv))
        else:
            self.h.decode_step(layer, qi, qa, out)
        # the inputs stay alive until the device has synchronized
        self._keep.append((qi, qa))
        return out

    def result(self, out, want_keys=False) -> StepResult:
        """The last step's results (after a device synchronize)."""
        sko = self.sko
        self._keep.clear()
        r = StepResult(topk=self.h.step_buffer(sko.SKO_BUF_TOPK), phys=self.h.step_buffer(sko.SKO_BUF_PHYS),
                       counts=self.h.step_buffer(sko.SKO_BUF_COUNTS), misses=self.h.step_buffer(sko.SKO_BUF_MISSES),
                       victims=self.h.step_buffer(sko.SKO_BUF_VICTIMS),
                       evict_old=self.h.step_buffer(sko.SKO_BUF_EVICT_OLD), out=out.cpu().numpy())
        if want_keys:
            r.keys = self.h.step_buffer(sko.SKO_BUF_KEYS)
        return r

    def decode(self, layer: int, q_idx: np.ndarray, q_attn: np.ndarray, want_keys=False) -> StepResult:
        out = self.issue(layer, q_idx, q_attn)
        self.torch.cuda.synchronize()
        return self.result(out, want_keys)

    def tables(self, layer: int, seq: int) -> Dict[str, np.ndarray]:
        sko = self.sko
        t = {"cache_slots": self.h.table(layer, seq, sko.SKO_TAB_CACHE_SLOTS),
             "slot_token": self.h.table(layer, seq, sko.SKO_TAB_SLOT_TOKEN),
             "last_use": self.h.table(layer, seq, sko.SKO_TAB_LAST_USE),
             "hot": self.h.table(layer, seq, sko.SKO_TAB_HOT)}
        # the device rows: each slot in its own row, the rest spare
        rows = np.concatenate([self.h.table(layer, seq, sko.SKO_TAB_SLOT_ROW),
                               self.h.table(layer, seq, sko.SKO_TAB_SPARE_ROWS)])
        assert np.array_equal(np.sort(rows), np.arange(rows.size)), \
            f"layer {layer} seq {seq}: slot and spare rows are not a permutation of the device rows"
        if self.h.cfg.flags & sko.SKO_FLAG_INDEXER_C8:
            t["idx_codes"] = self.h.table(layer, seq, sko.SKO_TAB_INDEXER)
            t["idx_scales"] = self.h.table(layer, seq, sko.SKO_TAB_INDEXER_SCALE)
        return t


class OracleSide:
    """The CPU oracle over a subset of (layer, seq) chains (each independent)."""

    def __init__(self, w: synth.Workload, chains: List[tuple], indexer_c8: bool = False):
        self.w = w
        self.chains = chains
        self.c8 = indexer_c8
        self.o = {c: oracle.Oracle(1, 1, w.capacity, w.top_k, w.hot_slots, w.positions, w.heads, SCALE,
                                   indexer_c8=indexer_c8)
                  for c in chains}

    def load_prefix(self, layer: int, seq: int) -> None:
        n = self.w.seq_context(seq)
        if n:
            self.o[(layer, seq)].append(0, 0, self.w.index_rows(layer, seq, 0, n), self.w.kv_rows(layer, seq, 0, n))

    def append_token(self, layer: int, seq: int, t: int) -> None:
        r = self.w.seq_context(seq) + t
        self.o[(layer, seq)].append(0, 0, self.w.index_rows(layer, seq, r, 1), self.w.kv_rows(layer, seq, r, 1))

    def decode(self, layer: int, seq: int, q_idx: np.ndarray, q_attn: np.ndarray, want_out=True,
               want_keys=False) -> dict:
        return self.o[(layer, seq)].decode_step(0, q_idx[None], q_attn[None], want_keys=want_keys,
                                                want_out=want_out)

    def tables(self, layer: int, seq: int) -> Dict[str, np.ndarray]:
        t = self.o[(layer, seq)].state(0, 0)
        if self.c8:
            t["idx_codes"], t["idx_scales"] = self.o[(layer, seq)].indexer_c8(0, 0)
        return t


def _sorted_by_token(packed: np.ndarray, other: Optional[np.ndarray] = None):
    tok = packed & 0x7FFFFFFF
    order = np.argsort(tok, kind="stable")
    return packed[order], (other[order] if other is not None else None)


def compare_step(w: synth.Workload, g: StepResult, seq: int, o: dict, check_out: bool = True,
                 where: str = "") -> Dict[str, float]:
    """Assert parity of one (seq) of a GPU step against the oracle's step."""
    cn_o = o["counts"][0]
    cn_g = g.counts[seq]
    assert np.array_equal(cn_g, cn_o), f"{where} counts gpu={cn_g.tolist()} oracle={cn_o.tolist()}"
    kk = int(cn_o[4])
    for p in range(w.positions):
        gw, gp = _sorted_by_token(g.topk[seq, p, :kk], g.phys[seq, p, :kk])
        ow, op = _sorted_by_token(o["topk"][0, p, :kk], o["phys"][0, p, :kk])
        if not np.array_equal(gw, ow):
            bad = np.nonzero(gw != ow)[0][:8]
            raise AssertionError(f"{where} topk p={p} differs at {bad.tolist()}: gpu={gw[bad].tolist()} oracle={ow[bad].tolist()}")
        assert np.array_equal(gp, op), f"{where} phys p={p} differs"
    nM = int(cn_o[2])
    for name in ("misses", "victims", "evict_old"):
        assert np.array_equal(getattr(g, name)[seq, :nM], o[name][0, :nM]), f"{where} {name} differs"
    stats = {}
    if check_out and "out" in o:
        go = g.out[seq].astype(np.float64)
        oo = o["out"][0]
        err = np.abs(go - oo)
        assert err.max() <= ATTN_ABS_TOL, f"{where} attention abs err {err.max():.3e}"
        if kk > 0:
            num = np.sqrt(np.mean((go - oo) ** 2, axis=-1))
            den = np.sqrt(np.mean(oo ** 2, axis=-1)) + 1e-30
            rel = num / den
            assert rel.max() <= ATTN_REL_RMS, f"{where} attention rel-RMS {rel.max():.3e}"
            stats["rel_rms"] = float(rel.max())
        stats["abs"] = float(err.max())
    if "keys" in o and g.keys is not None:
        Lt = int(cn_o[5])
        for p in range(w.positions):
            assert np.array_equal(g.keys[seq, p, :Lt], o["keys"][0, p, :Lt]), f"{where} score keys p={p} differ"
    return stats


def compare_tables(gt: Dict[str, np.ndarray], ot: Dict[str, np.ndarray], where: str = "") -> None:
    for name in ("cache_slots", "slot_token", "last_use"):
        if not np.array_equal(gt[name], ot[name]):
            bad = np.nonzero(gt[name] != ot[name])[0][:8]
            raise AssertionError(f"{where} table {name} differs at {bad.tolist()}")
    assert np.array_equal(gt["hot"], ot["hot"]), f"{where} hot-buffer bytes differ"
    if "idx_codes" in ot:
        # int8 indexer rows: codes and fp16 scale bits exactly
        for name in ("idx_codes", "idx_scales"):
            if not np.array_equal(gt[name], ot[name]):
                bad = np.unique(np.nonzero(gt[name] != ot[name])[0])[:8]
                raise AssertionError(f"{where} {name} differ at tokens {bad.tolist()}")


def run_parity(w: synth.Workload, layers: Optional[int] = None, steps: Optional[int] = None,
               chains: Optional[List[tuple]] = None, check_tables_every: int = 1,
               check_keys: bool = False, device_append: bool = True, out_steps=None,
               log=None, flags: int = 0, fused_append: bool = False) -> Dict[str, float]:
    """Run the full workload on the GPU; check the sampled chains on the CPU."""
    L = w.layers if layers is None else layers
    T = w.steps if steps is None else steps
    chains = [(l, b) for l in range(L) for b in range(w.batch)] if chains is None else chains
    inputs = Inputs(w, sorted({c[0] for c in chains} | set(range(L))), T)
    import sparse_kv_offload_amd as sko
    gpu = GpuSide(w, L, device_append=device_append,
                  flags=flags | (sko.SKO_FLAG_KEEP_KEYS if check_keys else 0), fused_append=fused_append)
    ora = OracleSide(w, chains, indexer_c8=bool(flags & sko.SKO_FLAG_INDEXER_C8))
    worst = {"abs": 0.0, "rel_rms": 0.0, "rescans": 0}
    try:
        for l in range(L):
            for b in range(w.batch):
                gpu.load_prefix(l, b)
        for c in chains:
            ora.load_prefix(*c)
        seqs = list(range(w.batch))
        for t in range(T):
            for l in range(L):
                gpu.append_token(l, t)
                qi = inputs.q_idx_step(l, t, seqs)
                qa = inputs.q_attn_step(l, t, seqs)
                g = gpu.decode(l, qi, qa, want_keys=check_keys)
                for (cl, b) in chains:
                    if cl != l:
                        continue
                    ora.append_token(l, b, t)
                    want_out = out_steps is None or t in out_steps
                    o = ora.decode(l, b, qi[b], qa[b], want_out=want_out, want_keys=check_keys)
                    s = compare_step(w, g, b, o, check_out=want_out, where=f"[{w.name} l={l} b={b} t={t}]")
                    for k_, v in s.items():
                        worst[k_] = max(worst[k_], v)
                    if check_tables_every and (t % check_tables_every == 0 or t == T - 1):
                        compare_tables(gpu.tables(l, b), ora.tables(l, b), where=f"[{w.name} l={l} b={b} t={t}]")
            if log:
                log(f"{w.name}: step {t + 1}/{T} ok")
        worst["rescans"] = sum(gpu.h.stats(l).rescans for l in range(L))
        if flags & sko.SKO_FLAG_SELECT_RESCAN:
            # every row with at least one token took the rescan path
            rows = sum(1 for b in range(w.batch) for t in range(T) if w.seq_context(b) + t + 1 > 0) * w.positions
            assert worst["rescans"] == L * rows, (worst["rescans"], L * rows)
    finally:
        gpu.close()
    return worst


def run_parity_micro(w: synth.Workload, nmb: int = 2, layers: Optional[int] = None, steps: Optional[int] = None,
                     chains: Optional[List[tuple]] = None, check_tables_every: int = 1,
                     fused_append: bool = True, out_steps=None, flags: int = 0, sync_each_layer: bool = True,
                     log=None) -> Dict[str, float]:
    """The batch split into nmb handles (contiguous groups of sequences), each
    kept off the copy blocks' XCD (SKO_FLAG_XCD_SPLIT) and on its own stream.
    Every layer-step queues all groups' calls before waiting, so the groups'
    steps overlap on the device.  With sync_each_layer every step of every
    sampled chain is checked against the oracle; without it the whole run is
    queued with no wait at all and the last step and the tables at the end
    are checked."""
    import sparse_kv_offload_amd as sko
    torch = torch_mod()
    L = w.layers if layers is None else layers
    T = w.steps if steps is None else steps
    chains = [(l, b) for l in range(L) for b in range(w.batch)] if chains is None else chains
    chain_set = set(chains)
    inputs = Inputs(w, sorted({c[0] for c in chains} | set(range(L))), T)
    groups = [list(range(g * w.batch // nmb, (g + 1) * w.batch // nmb)) for g in range(nmb)]
    assert all(groups), "every group needs a sequence"
    streams = [torch.cuda.Stream() for _ in groups]
    gpus = []
    worst = {"abs": 0.0, "rel_rms": 0.0}
    try:
        for grp, st in zip(groups, streams):
            gpus.append(GpuSide(w, L, flags=flags | sko.SKO_FLAG_XCD_SPLIT, fused_append=fused_append,
                                seqs=grp, stream=st))
        for gs in gpus:
            for l in range(L):
                for j in range(len(gs.seqs)):
                    gs.load_prefix(l, j)
        torch.cuda.synchronize()
        ora = OracleSide(w, chains, indexer_c8=bool(flags & sko.SKO_FLAG_INDEXER_C8))
        for c in chains:
            ora.load_prefix(*c)

        def check(gs, out, l, t, tables_now):
            g = gs.result(out)
            for j, b in enumerate(gs.seqs):
                if (l, b) not in chain_set:
                    continue
                want_out = out_steps is None or t in out_steps
                o = ora.decode(l, b, inputs.q_idx[(l, b)][t], inputs.w.attn_queries(l, b, t), want_out=want_out)
                s_ = compare_step(w, g, j, o, check_out=want_out, where=f"[{w.name} micro{nmb} l={l} b={b} t={t}]")
                for k_, v in s_.items():
                    worst[k_] = max(worst[k_], v)
                if tables_now:
                    compare_tables(gs.tables(l, j), ora.tables(l, b), where=f"[{w.name} micro{nmb} l={l} b={b} t={t}]")

        for t in range(T):
            for l in range(L):
                outs = []
                for gs in gpus:
                    gs.append_token(l, t)
                    outs.append(gs.issue(l, inputs.q_idx_step(l, t, gs.seqs), inputs.q_attn_step(l, t, gs.seqs)))
                if sync_each_layer:
                    torch.cuda.synchronize()
                    for gs, out in zip(gpus, outs):
                        for b in gs.seqs:
                            if (l, b) in chain_set:
                                ora.append_token(l, b, t)
                        tables_now = bool(check_tables_every) and (t % check_tables_every == 0 or t == T - 1)
                        check(gs, out, l, t, tables_now)
                else:
                    last = outs
                    for b in range(w.batch):
                        if (l, b) in chain_set:
                            ora.append_token(l, b, t)
                            if not (t == T - 1 and l == L - 1):
                                ora.decode(l, b, inputs.q_idx[(l, b)][t], inputs.w.attn_queries(l, b, t),
                                           want_out=False)
            if log:
                log(f"{w.name} micro{nmb}: step {t + 1}/{T} queued")
        if not sync_each_layer:
            torch.cuda.synchronize()
            for gs, out in zip(gpus, last):
                check(gs, out, L - 1, T - 1, True)
            # every other layer's tables after the whole run
            for gs in gpus:
                for j, b in enumerate(gs.seqs):
                    for l in range(L - 1):
                        if (l, b) in chain_set:
                            compare_tables(gs.tables(l, j), ora.tables(l, b), where=f"[{w.name} micro{nmb} end l={l} b={b}]")
    finally:
        torch.cuda.synchronize()
        for gs in gpus:
            gs.close()
    return worst
