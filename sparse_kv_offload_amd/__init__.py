"""Python binding of libsko, the sparse decode offload step for MI355X.

Argument marshalling only: every stage of the step runs in the HIP kernels of
``libsko.so`` (built from ``csrc/`` by ``build.py``).  The functions carry the
names of the C ABI in ``include/sko.h``; :class:`SparseKVOffload` is a small
convenience wrapper over them.  Buffers may be given as torch tensors (device
or host), numpy arrays (host) or raw integer addresses.  PyTorch only
provides device memory and the stream.

There is no fallback: if the library is missing, importing this package
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsko.so")

SKO_OK = 0
SKO_E_INVAL = -1
SKO_E_NOMEM = -2
SKO_E_DEVICE = -3
SKO_E_CAPACITY = -4
SKO_E_STATE = -5
SKO_E_UNSUPPORTED = -6
SKO_ALL_SEQS = -1
SKO_INDEX_DIM, SKO_KV_DIM, SKO_V_DIM = 64, 576, 512
SKO_MAX_MERGE = 8192
SKO_FLAG_POOL_COHERENT = 0x1
SKO_FLAG_POOL_NONCOHERENT = 0x2
SKO_FLAG_KEEP_KEYS = 0x4
SKO_FLAG_SELECT_RESCAN = 0x8
SKO_FLAG_FUSED_COPY = 0x10
SKO_FLAG_LATE_COPY = 0x20
SKO_FLAG_EARLY_COPY = 0x40
SKO_FLAG_INDEXER_C8 = 0x80
SKO_FLAG_HIT_OVERLAP = 0x100
SKO_FLAG_TEST_VIOLATION = 0x200
SKO_FLAG_XCD_SPLIT = 0x400

SKO_BUF_TOPK, SKO_BUF_PHYS, SKO_BUF_COUNTS = 1, 2, 3
SKO_BUF_MISSES, SKO_BUF_VICTIMS, SKO_BUF_EVICT_OLD, SKO_BUF_KEYS = 4, 5, 6, 7
SKO_TAB_CACHE_SLOTS, SKO_TAB_SLOT_TOKEN, SKO_TAB_LAST_USE = 1, 2, 3
SKO_TAB_HOT, SKO_TAB_INDEXER, SKO_TAB_POOL, SKO_TAB_NTOK = 4, 5, 6, 7
SKO_TAB_INDEXER_SCALE = 8
SKO_TAB_SLOT_ROW, SKO_TAB_SPARE_ROWS = 9, 10

EXPORTED = (
    "sko_create", "sko_set_stream", "sko_append_token", "sko_decode_step", "sko_decode_step_static",
    "sko_decode_step_append",
    "sko_read_step",
    "sko_read_table", "sko_get_stats", "sko_set_timing", "sko_get_timing", "sko_get_copy_overlap",
    "sko_get_copy_spans", "sko_stage_name",
    "sko_num_stages", "sko_destroy", "sko_last_error", "sko_version", "sko_link_read_rate", "sko_hbm_gather_rate",
    "sko_hbm_read_rate",
    # layerwise prefill offload (include/sko_prefill.h)
    "sko_prefill_plan", "sko_prefill_create", "sko_prefill_destroy", "sko_prefill_host_pool",
    "sko_prefill_set_tokens", "sko_prefill_begin_layer", "sko_prefill_end_layer", "sko_prefill_sync",
    "sko_prefill_layer_timing", "sko_prefill_get_plan",
)


class SkoConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
        ("index_dim", ctypes.c_int32),
        ("kv_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hot_slots", ctypes.c_int32),
        ("mtp_positions", ctypes.c_int32),
        ("attn_scale", ctypes.c_float),
        ("device", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class SkoPrefillConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("shared_buffers", ctypes.c_int32),
        ("lookahead", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
        ("capacity_tokens", ctypes.c_int64),
        ("device", ctypes.c_int32),
        ("independent", ctypes.c_void_p),
    ]


class SkoSeqCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("unique", "hits", "misses", "evictions", "selected", "tokens", "step", "reserved")]


class SkoLayerStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("steps", "unique", "hits", "misses", "evictions", "h2d_bytes", "rescans", "direct_rows")]


class SkoError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed ({code}): {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libsko.so not found at {LIB_PATH}; build it first "
            "(python sparse_kv_offload_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "sko_create": (ctypes.c_int, [ctypes.POINTER(SkoConfig), vp, ctypes.POINTER(vp)]),
        "sko_set_stream": (ctypes.c_int, [vp, vp]),
        "sko_append_token": (ctypes.c_int, [vp, i32, i32, vp, vp, i64, i32]),
        "sko_decode_step": (ctypes.c_int, [vp, i32, vp, vp, vp]),
        "sko_decode_step_static": (ctypes.c_int, [vp, i32, vp, vp, vp]),
        "sko_decode_step_append": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp]),
        "sko_read_step": (ctypes.c_int, [vp, i32, vp, i64]),
        "sko_read_table": (ctypes.c_int, [vp, i32, i32, i32, vp, i64]),
        "sko_get_stats": (ctypes.c_int, [vp, i32, ctypes.POINTER(SkoLayerStats)]),
        "sko_set_timing": (ctypes.c_int, [vp, ctypes.c_uint32]),
        "sko_get_timing": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64), i32]),
        "sko_get_copy_overlap": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "sko_get_copy_spans": (ctypes.c_int, [vp, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]),
        "sko_stage_name": (ctypes.c_char_p, [i32]),
        "sko_num_stages": (i32, []),
        "sko_destroy": (None, [vp]),
        "sko_last_error": (ctypes.c_char_p, []),
        "sko_version": (ctypes.c_char_p, []),
        "sko_link_read_rate": (ctypes.c_int, [i32, i64, i32, ctypes.POINTER(ctypes.c_float)]),
        "sko_hbm_gather_rate": (ctypes.c_int, [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_float)]),
        "sko_hbm_read_rate": (ctypes.c_int, [i32, i64, i32, ctypes.POINTER(ctypes.c_float)]),
        "sko_prefill_plan": (ctypes.c_int, [i32, vp, vp, i32, vp, vp, vp]),
        "sko_prefill_create": (ctypes.c_int, [ctypes.POINTER(SkoPrefillConfig), vp, ctypes.POINTER(vp)]),
        "sko_prefill_destroy": (ctypes.c_int, [vp]),
        "sko_prefill_host_pool": (ctypes.c_int, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(i64)]),
        "sko_prefill_set_tokens": (ctypes.c_int, [vp, i32, i64]),
        "sko_prefill_begin_layer": (ctypes.c_int, [vp, i32, ctypes.POINTER(vp)]),
        "sko_prefill_end_layer": (ctypes.c_int, [vp, i32, i64]),
        "sko_prefill_sync": (ctypes.c_int, [vp]),
        "sko_prefill_layer_timing": (ctypes.c_int, [vp, i32, ctypes.POINTER(ctypes.c_float),
                                                    ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
        "sko_prefill_get_plan": (ctypes.c_int, [vp, vp, ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _addr(x) -> Optional[int]:
    """Raw address of a torch tensor, numpy array or integer."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy buffers must be C-contiguous")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot take the address of {type(x)!r}")


def _is_device(x) -> bool:
    return hasattr(x, "is_cuda") and bool(x.is_cuda)


def _check(rc: int, where: str) -> None:
    if rc != SKO_OK:
        raise SkoError(rc, where, sko_last_error())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# --------------------------------------------------------------- C ABI names

def sko_last_error() -> str:
    return (_lib.sko_last_error() or b"").decode()


def sko_version() -> str:
    return _lib.sko_version().decode()


def sko_link_read_rate(device: int = 0, nbytes: int = 1 << 30, reps: int = 3) -> float:
    """Host-link read rate (GB/s) of a streaming kernel over pinned host memory."""
    v = ctypes.c_float()
    _check(_lib.sko_link_read_rate(device, nbytes, reps, ctypes.byref(v)), "sko_link_read_rate")
    return float(v.value)


def sko_hbm_gather_rate(device: int = 0, seqs: int = 32, slots: int = 8192, rows_per_seq: int = 2048,
                        reps: int = 3) -> float:
    """HBM read rate (GB/s) of random whole-row gathers, the attention's pattern."""
    v = ctypes.c_float()
    _check(_lib.sko_hbm_gather_rate(device, seqs, slots, rows_per_seq, reps, ctypes.byref(v)),
           "sko_hbm_gather_rate")
    return float(v.value)


def sko_hbm_read_rate(device: int = 0, nbytes: int = 1 << 28, reps: int = 5) -> float:
    """HBM rate (GB/s) of a plain streaming read, the indexer score pass's pattern."""
    v = ctypes.c_float()
    _check(_lib.sko_hbm_read_rate(device, nbytes, reps, ctypes.byref(v)), "sko_hbm_read_rate")
    return float(v.value)


def sko_num_stages() -> int:
    return int(_lib.sko_num_stages())


def sko_stage_name(stage: int) -> str:
    return (_lib.sko_stage_name(stage) or b"").decode()


def sko_create(cfg: SkoConfig, stream=None) -> int:
    h = ctypes.c_void_p()
    _check(_lib.sko_create(ctypes.byref(cfg), _stream_handle(stream), ctypes.byref(h)), "sko_create")
    return int(h.value)


def sko_set_stream(h: int, stream) -> None:
    _check(_lib.sko_set_stream(h, _stream_handle(stream)), "sko_set_stream")


def sko_append_token(h: int, layer: int, seq: int, idx_rows, kv_rows, n: int,
                     src_on_device: Optional[bool] = None) -> None:
    dev = _is_device(idx_rows) if src_on_device is None else bool(src_on_device)
    _check(_lib.sko_append_token(h, layer, seq, _addr(idx_rows), _addr(kv_rows), n, int(dev)),
           "sko_append_token")


def sko_decode_step(h: int, layer: int, q_idx, q_attn, out) -> None:
    _check(_lib.sko_decode_step(h, layer, _addr(q_idx), _addr(q_attn), _addr(out)), "sko_decode_step")


def sko_decode_step_append(h: int, layer: int, idx_rows, kv_rows, q_idx, q_attn, out) -> None:
    """Append one token per sequence (device rows) and decode, in one call."""
    _check(_lib.sko_decode_step_append(h, layer, _addr(idx_rows), _addr(kv_rows), _addr(q_idx), _addr(q_attn),
                                       _addr(out)), "sko_decode_step_append")


def sko_decode_step_static(h: int, layer: int, q_idx, q_attn, out) -> None:
    _check(_lib.sko_decode_step_static(h, layer, _addr(q_idx), _addr(q_attn), _addr(out)),
           "sko_decode_step_static")


def sko_read_step(h: int, which: int, dst: np.ndarray) -> np.ndarray:
    _check(_lib.sko_read_step(h, which, _addr(dst), dst.nbytes), "sko_read_step")
    return dst


def sko_read_table(h: int, layer: int, seq: int, which: int, dst: np.ndarray) -> np.ndarray:
    _check(_lib.sko_read_table(h, layer, seq, which, _addr(dst), dst.nbytes), "sko_read_table")
    return dst


def sko_get_stats(h: int, layer: int) -> SkoLayerStats:
    st = SkoLayerStats()
    _check(_lib.sko_get_stats(h, layer, ctypes.byref(st)), "sko_get_stats")
    return st


def sko_set_timing(h: int, stage_mask) -> None:
    """stage_mask: int bit mask, True (all stages) or False/0 (off)."""
    if stage_mask is True:
        stage_mask = 0xFFFFFFFF
    _check(_lib.sko_set_timing(h, int(stage_mask) & 0xFFFFFFFF), "sko_set_timing")


def sko_stage_index(name: str) -> int:
    for i in range(sko_num_stages()):
        if sko_stage_name(i) == name:
            return i
    raise KeyError(name)


def sko_get_timing(h: int) -> dict:
    n = sko_num_stages()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(_lib.sko_get_timing(h, ms, cnt, n), "sko_get_timing")
    return {sko_stage_name(i): (float(ms[i]), int(cnt[i])) for i in range(n)}


def sko_get_copy_overlap(h: int) -> dict:
    """Sums over the recorded LRU-update launches: copy span, merge span and
    their overlap (ms), and the number of launches."""
    c, m, o, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(_lib.sko_get_copy_overlap(h, ctypes.byref(c), ctypes.byref(m), ctypes.byref(o), ctypes.byref(n)),
           "sko_get_copy_overlap")
    return {"copy_ms": c.value, "merge_ms": m.value, "overlap_ms": o.value, "launches": n.value}


def sko_get_copy_spans(h: int) -> tuple:
    """(spans [n][2] uint64 device-clock ticks, clock_khz) of the recorded
    LRU-update launches' copy spans."""
    n, khz = ctypes.c_int32(), ctypes.c_double()
    _check(_lib.sko_get_copy_spans(h, None, 0, ctypes.byref(n), ctypes.byref(khz)), "sko_get_copy_spans")
    a = np.zeros((max(n.value, 1), 2), dtype=np.uint64)
    _check(_lib.sko_get_copy_spans(h, _addr(a), n.value, ctypes.byref(n), ctypes.byref(khz)), "sko_get_copy_spans")
    return a[:n.value].copy(), khz.value


def sko_destroy(h: int) -> None:
    if h:
        _lib.sko_destroy(h)


def make_config(*, num_layers: int, batch: int, max_tokens: int, num_heads: int, top_k: int,
                hot_slots: int, mtp_positions: int = 1, attn_scale: float = 1.0 / 24.0,
                device: int = 0, index_dim: int = SKO_INDEX_DIM, kv_dim: int = SKO_KV_DIM,
                v_dim: int = SKO_V_DIM, flags: int = 0) -> SkoConfig:
    return SkoConfig(num_layers, batch, max_tokens, index_dim, kv_dim, v_dim, num_heads, top_k,
                     hot_slots, mtp_positions, attn_scale, device, flags)


class SparseKVOffload:
    """Owner of one libsko handle (thin convenience over the C ABI)."""

    def __init__(self, cfg: SkoConfig, stream=None):
        self.cfg = cfg
        self.handle = sko_create(cfg, stream)

    def close(self) -> None:
        if self.handle:
            sko_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, layer: int, seq: int, idx_rows, kv_rows, n: Optional[int] = None) -> None:
        if n is None:
            rows = idx_rows.shape[0]
            n = rows if seq != SKO_ALL_SEQS else rows // self.cfg.batch
        sko_append_token(self.handle, layer, seq, idx_rows, kv_rows, n)

    def decode_step(self, layer: int, q_idx, q_attn, out) -> None:
        sko_decode_step(self.handle, layer, q_idx, q_attn, out)

    def decode_step_append(self, layer: int, idx_rows, kv_rows, q_idx, q_attn, out) -> None:
        sko_decode_step_append(self.handle, layer, idx_rows, kv_rows, q_idx, q_attn, out)

    # ---- inspection ----
    def step_buffer(self, which: int) -> np.ndarray:
        c = self.cfg
        B, D, k = c.batch, c.mtp_positions, c.top_k
        if which == SKO_BUF_COUNTS:
            a = np.zeros((B, 8), dtype=np.int32)
        elif which in (SKO_BUF_TOPK, SKO_BUF_PHYS):
            a = np.zeros((B, D, k), dtype=np.int32)
        elif which == SKO_BUF_KEYS:
            a = np.zeros((B, D, c.max_tokens), dtype=np.uint32)
        else:
            a = np.zeros((B, D * k), dtype=np.int32)
        return sko_read_step(self.handle, which, a)

    def table(self, layer: int, seq: int, which: int) -> np.ndarray:
        c = self.cfg
        shapes = {
            SKO_TAB_CACHE_SLOTS: ((c.max_tokens,), np.int32),
            SKO_TAB_SLOT_TOKEN: ((c.hot_slots,), np.int32),
            SKO_TAB_LAST_USE: ((c.hot_slots,), np.int32),
            SKO_TAB_HOT: ((c.hot_slots, SKO_KV_DIM), np.uint16),
            SKO_TAB_INDEXER: ((c.max_tokens, SKO_INDEX_DIM),
                              np.int8 if c.flags & SKO_FLAG_INDEXER_C8 else np.uint16),
            SKO_TAB_POOL: ((c.max_tokens, SKO_KV_DIM), np.uint16),
            SKO_TAB_NTOK: ((1,), np.int64),
            SKO_TAB_INDEXER_SCALE: ((c.max_tokens,), np.uint16),
            SKO_TAB_SLOT_ROW: ((c.hot_slots,), np.int32),
            SKO_TAB_SPARE_ROWS: ((c.mtp_positions * c.top_k,), np.int32),
        }
        shape, dt = shapes[which]
        return sko_read_table(self.handle, layer, seq, which, np.zeros(shape, dtype=dt))

    def stats(self, layer: int) -> SkoLayerStats:
        return sko_get_stats(self.handle, layer)

    def set_timing(self, stage_mask) -> None:
        sko_set_timing(self.handle, stage_mask)

    def timing(self) -> dict:
        return sko_get_timing(self.handle)

    def copy_overlap(self) -> dict:
        return sko_get_copy_overlap(self.handle)

    def copy_spans(self):
        return sko_get_copy_spans(self.handle)


__all__ = [n for n in globals() if n.startswith(("sko_", "SKO_", "Sko"))] + [
    "SparseKVOffload", "make_config", "LIB_PATH", "EXPORTED"]


# ------------------------------------------------------------ prefill offload

def sko_prefill_plan(specs, independent, shared: int, layer_bytes):
    """Buffer of every layer and the number of physical buffers."""
    n = len(specs)
    sp = np.ascontiguousarray(specs, dtype=np.int32)
    ind = np.ascontiguousarray(independent, dtype=np.int32)
    lb = np.ascontiguousarray(layer_bytes, dtype=np.int64)
    if ind.size != n or lb.size != n:
        raise ValueError("specs, independent and layer_bytes need one entry per layer")
    out = np.zeros(max(n, 1), dtype=np.int32)
    nphys = ctypes.c_int32(0)
    _check(_lib.sko_prefill_plan(n, _addr(sp), _addr(ind), int(shared), _addr(lb), _addr(out),
                                 ctypes.byref(nphys)), "sko_prefill_plan")
    return out[:n].copy(), int(nphys.value)


def sko_prefill_create(cfg: SkoPrefillConfig, stream=None) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(_lib.sko_prefill_create(ctypes.byref(cfg), _stream_handle(stream), ctypes.byref(h)),
           "sko_prefill_create")
    return h


def sko_prefill_destroy(h) -> None:
    _lib.sko_prefill_destroy(h)


def sko_prefill_host_pool(h, layer: int):
    """(host address of the layer's rows, tokens held)."""
    p, t = ctypes.c_void_p(), ctypes.c_int64()
    _check(_lib.sko_prefill_host_pool(h, layer, ctypes.byref(p), ctypes.byref(t)), "sko_prefill_host_pool")
    return int(p.value), int(t.value)


def sko_prefill_set_tokens(h, layer: int, tokens: int) -> None:
    _check(_lib.sko_prefill_set_tokens(h, layer, tokens), "sko_prefill_set_tokens")


def sko_prefill_begin_layer(h, layer: int) -> int:
    p = ctypes.c_void_p()
    _check(_lib.sko_prefill_begin_layer(h, layer, ctypes.byref(p)), "sko_prefill_begin_layer")
    return int(p.value)


def sko_prefill_end_layer(h, layer: int, new_tokens: int) -> None:
    _check(_lib.sko_prefill_end_layer(h, layer, new_tokens), "sko_prefill_end_layer")


def sko_prefill_sync(h) -> None:
    _check(_lib.sko_prefill_sync(h), "sko_prefill_sync")


def sko_prefill_layer_timing(h, layer: int):
    a, w, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    _check(_lib.sko_prefill_layer_timing(h, layer, ctypes.byref(a), ctypes.byref(w), ctypes.byref(c)),
           "sko_prefill_layer_timing")
    return float(a.value), float(w.value), float(c.value)


def sko_prefill_get_plan(h, num_layers: int):
    out = np.zeros(num_layers, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(_lib.sko_prefill_get_plan(h, _addr(out), ctypes.byref(n)), "sko_prefill_get_plan")
    return out, int(n.value)


class PrefillOffload:
    """Owns one sko_prefill_handle (include/sko_prefill.h)."""

    def __init__(self, num_layers: int, shared_buffers: int, lookahead: int, row_bytes: int,
                 capacity_tokens: int, independent=None, stream=None, device: int = 0):
        self._ind = None if independent is None else np.ascontiguousarray(independent, dtype=np.int32)
        cfg = SkoPrefillConfig(num_layers, shared_buffers, lookahead, row_bytes, capacity_tokens, device,
                               None if self._ind is None else self._ind.ctypes.data)
        self.handle = sko_prefill_create(cfg, stream)
        self.num_layers, self.row_bytes, self.capacity = num_layers, row_bytes, capacity_tokens

    def close(self) -> None:
        if self.handle:
            sko_prefill_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def host_pool(self, layer: int) -> np.ndarray:
        """The layer's pinned host rows as a numpy view [capacity][row_bytes] (uint8)."""
        addr, _ = sko_prefill_host_pool(self.handle, layer)
        buf = (ctypes.c_uint8 * (self.capacity * self.row_bytes)).from_address(addr)
        return np.frombuffer(buf, dtype=np.uint8).reshape(self.capacity, self.row_bytes)

    def tokens(self, layer: int) -> int:
        return sko_prefill_host_pool(self.handle, layer)[1]

    def set_tokens(self, layer: int, tokens: int) -> None:
        sko_prefill_set_tokens(self.handle, layer, tokens)

    def begin_layer(self, layer: int) -> int:
        """Device address of the layer's buffer (its KV first)."""
        return sko_prefill_begin_layer(self.handle, layer)

    def end_layer(self, layer: int, new_tokens: int) -> None:
        sko_prefill_end_layer(self.handle, layer, new_tokens)

    def sync(self) -> None:
        sko_prefill_sync(self.handle)

    def layer_timing(self, layer: int):
        """(load_ms, exposed_ms, compute_ms) of the layer in the last pass."""
        return sko_prefill_layer_timing(self.handle, layer)

    def plan(self):
        return sko_prefill_get_plan(self.handle, self.num_layers)
