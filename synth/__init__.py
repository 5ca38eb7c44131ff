"""Seeded synthetic inputs for the sparse decode offload step.

Test and benchmark infrastructure: the one input source that the CPU oracle
and the HIP path both consume.  Nothing here computes any part of the decode
method; it draws keys, rows and queries with the shapes and distributions of
the workloads and hands them out as raw bf16 bit patterns (numpy uint16).

Workload recipe (stated once here, mirrored in the design notes):
  * indexer keys: 64 x bf16 per token, i.i.d. N(0, 1);
  * main-KV rows: 576 x bf16 per token (512 latent + 64 rope), i.i.d. N(0, 1);
  * indexer query chain per (layer, seq): q_0 = normalize(z_0),
    q_t = normalize(a * q_{t-1} + c * z_t); at a topic-jump step the chain
    restarts from normalize(z_t); the chain is kept in float64 and rounded
    to bf16 (via float32) only on output;
  * D > 1 query positions: position p uses q_t + noise * zeta_{t,p} (not
    re-normalised); D = 1 uses q_t itself;
  * attention queries: i.i.d. N(0, 1) bf16, 576 per (layer, seq, step,
    position, head).
All draws come from a counter-based SplitMix64 stream (synth.c), so any row
can be regenerated alone.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream kinds
KIND_INDEX_KEY = 1
KIND_KV_ROW = 2
KIND_QUERY_NOISE = 3
KIND_QUERY_POS = 4
KIND_ATTN_QUERY = 5

INDEX_DIM = 64
KV_DIM = 576
V_DIM = 512


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP for the bulk fills)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
    lib.synth_stream_key.restype = u64
    lib.synth_stream_key.argtypes = [u64, u32, u32, u32, u64]
    lib.synth_normal_f64.restype = None
    lib.synth_normal_f64.argtypes = [u64, u64, u64, u32, vp]
    lib.synth_normal_bf16.restype = None
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, u32, vp]
    lib.synth_raw_u64.restype = None
    lib.synth_raw_u64.argtypes = [u64, u64, u64, vp]
    lib.synth_splitmix64_sequence.restype = None
    lib.synth_splitmix64_sequence.argtypes = [u64, u64, vp]
    lib.synth_f64_to_bf16.restype = None
    lib.synth_f64_to_bf16.argtypes = [vp, u64, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_key(seed: int, kind: int, layer: int, seq: int, extra: int = 0) -> int:
    return int(_load().synth_stream_key(seed & (2**64 - 1), kind, layer, seq, extra))


def normal_f64(key: int, row0: int, nrows: int, width: int) -> np.ndarray:
    assert width % 2 == 0
    out = np.empty((nrows, width), dtype=np.float64)
    if nrows:
        _load().synth_normal_f64(key, row0, nrows, width, _ptr(out))
    return out


def normal_bf16(key: int, row0: int, nrows: int, width: int,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    assert width % 2 == 0
    if out is None:
        out = np.empty((nrows, width), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == nrows * width
    if nrows:
        _load().synth_normal_bf16(key, row0, nrows, width, _ptr(out))
    return out


def raw_u64(key: int, n0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_raw_u64(key, n0, n, _ptr(out))
    return out


def splitmix64_sequence(state: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_splitmix64_sequence(state, n, _ptr(out))
    return out


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_f64_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bit patterns to float32."""
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, step count and query recipe."""
    name: str
    layers: int
    batch: int
    context: int            # L0, tokens present before the first decode step
    steps: int              # T decode steps, one appended token each
    top_k: int
    hot_slots: int
    positions: int = 1      # D query positions per step (MTP3 = 4)
    heads: int = 16
    drift: Tuple[float, float] = (0.9, 0.1)
    jump_every: int = 0     # fresh query every N steps (0 = never)
    pos_noise: float = 0.05
    seed: int = 1234
    # per-sequence context override for ragged batches (None = all `context`)
    contexts: Optional[Tuple[int, ...]] = None

    @property
    def capacity(self) -> int:
        return max(self.seq_context(b) for b in range(self.batch)) + self.steps

    def seq_context(self, seq: int) -> int:
        return self.context if self.contexts is None else self.contexts[seq]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- rows -------------------------------------------------------------
    def index_rows(self, layer: int, seq: int, row0: int, n: int,
                   out: Optional[np.ndarray] = None) -> np.ndarray:
        key = stream_key(self.seed, KIND_INDEX_KEY, layer, seq)
        return normal_bf16(key, row0, n, INDEX_DIM, out)

    def kv_rows(self, layer: int, seq: int, row0: int, n: int,
                out: Optional[np.ndarray] = None) -> np.ndarray:
        key = stream_key(self.seed, KIND_KV_ROW, layer, seq)
        return normal_bf16(key, row0, n, KV_DIM, out)

    # ---- queries ----------------------------------------------------------
    def index_query_chain(self, layer: int, seq: int, steps: Optional[int] = None) -> np.ndarray:
        """float64 [T][D][64] position queries (before bf16 rounding)."""
        T = self.steps if steps is None else steps
        z = normal_f64(stream_key(self.seed, KIND_QUERY_NOISE, layer, seq), 0, T, INDEX_DIM)
        a, c = self.drift
        q = np.empty((T, INDEX_DIM), dtype=np.float64)
        for t in range(T):
            if t == 0 or (self.jump_every and t % self.jump_every == 0):
                v = z[t]
            else:
                v = a * q[t - 1] + c * z[t]
            q[t] = v / np.sqrt(np.dot(v, v))
        D = self.positions
        if D == 1:
            return q[:, None, :].copy()
        zeta = normal_f64(stream_key(self.seed, KIND_QUERY_POS, layer, seq), 0, T * D, INDEX_DIM)
        return q[:, None, :] + self.pos_noise * zeta.reshape(T, D, INDEX_DIM)

    def index_queries(self, layer: int, seq: int, steps: Optional[int] = None) -> np.ndarray:
        """bf16 [T][D][64]."""
        return f64_to_bf16(self.index_query_chain(layer, seq, steps))

    def attn_queries(self, layer: int, seq: int, step: int) -> np.ndarray:
        """bf16 [D][H][576]."""
        key = stream_key(self.seed, KIND_ATTN_QUERY, layer, seq, step)
        return normal_bf16(key, 0, self.positions * self.heads, KV_DIM).reshape(
            self.positions, self.heads, KV_DIM)


# The five workloads of the benchmark suite (sizes as described for the
# sparse decode offload step: tiny, small, MTP3 dedupe, shelf sweep, long).
TINY = Workload("tiny", layers=1, batch=1, context=4096, steps=8, top_k=256, hot_slots=512,
                positions=1, heads=1)
SMALL = Workload("small", layers=4, batch=8, context=32768, steps=64, top_k=2048,
                 hot_slots=4096, positions=1, heads=16)
MTP3 = Workload("mtp3", layers=4, batch=16, context=131072, steps=128, top_k=2048,
                hot_slots=16384, positions=4, heads=16)
SHELF8 = Workload("shelf_ctx8", layers=8, batch=32, context=65536, steps=256, top_k=2048,
                  hot_slots=8192, positions=1, heads=16, drift=(0.95, 0.05), jump_every=64)
SHELF4 = SHELF8.replace(name="shelf_ctx4", hot_slots=16384)
LONG = Workload("long", layers=2, batch=2, context=1048576, steps=64, top_k=2048,
                hot_slots=131072, positions=4, heads=16)

WORKLOADS = {w.name: w for w in (TINY, SMALL, MTP3, SHELF8, SHELF4, LONG)}
