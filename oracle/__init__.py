"""CPU oracle for the sparse decode offload step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product path under
``sparse_kv_offload_amd/`` never imports this package, and this package never
imports it.

The arithmetic lives in ``sko_oracle.cpp`` (plain single-threaded C++17,
compiled with g++, no fast-math, no FMA contraction beyond the explicit
``std::fma`` of the score).  See that file's header for the readings it takes
of the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sko_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

IDX_DIM, KV_DIM, V_DIM = 64, 576, 512

# planted-mistake switch values (must match the enum in sko_oracle.cpp)
MUTATIONS = {
    "score_drop_last_term": 1,
    "tie_larger_index": 2,
    "no_dedupe": 3,
    "victim_slot_desc": 4,
    "victim_ignore_stamp": 5,
    "scale_512": 6,
    "v_wrong_slice": 7,
    "hits_not_stamped": 8,
    "evict_keeps_old": 9,
    "flag_inverted": 10,
    "score_swap_operand": 11,
    "c8_hadamard_sign": 12,
    "c8_truncate": 13,
    "c8_query_not_rotated": 14,
    "c8_scale_255": 15,
    "c8_no_query_scale": 16,
    "step_victim_slot_desc": 17,
    "step_miss_desc": 18,
    "append_offset": 19,
}


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp]
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
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_set_mutation.argtypes = [i32]
    lib.oracle_set_mutation.restype = None
    lib.oracle_create.argtypes = [i32, i32, i64, i32, i32, i32, i32, f32]
    lib.oracle_create.restype = vp
    lib.oracle_destroy.argtypes = [vp]
    lib.oracle_destroy.restype = None
    lib.oracle_append.argtypes = [vp, i32, i32, vp, vp, i64]
    lib.oracle_append.restype = i32
    lib.oracle_decode_step.argtypes = [vp, i32, vp, vp] + [vp] * 9
    lib.oracle_decode_step.restype = i32
    lib.oracle_read_state.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_read_state.restype = i32
    lib.oracle_score_one.argtypes = [vp, vp]
    lib.oracle_score_one.restype = f32
    lib.oracle_ordered_key.argtypes = [f32]
    lib.oracle_ordered_key.restype = ctypes.c_uint32
    lib.oracle_topk.argtypes = [vp, i64, i32, vp]
    lib.oracle_topk.restype = i32
    lib.oracle_lru_apply.argtypes = [vp, i64, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.oracle_lru_apply.restype = i32
    lib.oracle_attention.argtypes = [vp, i32, vp, i32, f32, vp]
    lib.oracle_attention.restype = None
    lib.oracle_set_indexer_c8.argtypes = [vp, i32]
    lib.oracle_set_indexer_c8.restype = i32
    lib.oracle_read_indexer_c8.argtypes = [vp, i32, i32, vp, vp]
    lib.oracle_read_indexer_c8.restype = i32
    lib.oracle_hadamard_rotate.argtypes = [vp, vp]
    lib.oracle_hadamard_rotate.restype = None
    lib.oracle_quantize_row.argtypes = [vp, vp, vp]
    lib.oracle_quantize_row.restype = None
    lib.oracle_c8_score.argtypes = [vp, ctypes.c_uint16, vp, ctypes.c_uint16]
    lib.oracle_c8_score.restype = f32
    lib.oracle_f32_to_f16.argtypes = [f32]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = f32
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def set_mutation(name_or_id) -> None:
    """Plant a deliberate mistake (tests of the pins only); 0/None clears it."""
    mid = 0 if not name_or_id else (MUTATIONS[name_or_id] if isinstance(name_or_id, str) else int(name_or_id))
    _load().oracle_set_mutation(mid)


def score_one(q: np.ndarray, krow: np.ndarray) -> float:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    krow = np.ascontiguousarray(krow, dtype=np.uint16)
    assert q.size == IDX_DIM and krow.size == IDX_DIM
    return float(np.float32(_load().oracle_score_one(_p(q), _p(krow))))


def ordered_key(s: float) -> int:
    return int(_load().oracle_ordered_key(float(s)))


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    s = np.ascontiguousarray(scores, dtype=np.float32)
    out = np.empty(max(1, min(k, s.size)), dtype=np.int32)
    n = _load().oracle_topk(_p(s), s.size, k, _p(out))
    return out[:n].copy()


def attention(qa: np.ndarray, rows: np.ndarray, scale: float) -> np.ndarray:
    """qa [H][576] bf16, rows [n][576] bf16 -> [H][512] float64."""
    qa = np.ascontiguousarray(qa, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    H = qa.shape[0]
    out = np.empty((H, V_DIM), dtype=np.float64)
    _load().oracle_attention(_p(qa), H, _p(rows), rows.shape[0], scale, _p(out))
    return out


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """bf16 [64] -> binary32 [64]: (1/8) H x (int8-indexer rotation)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size == IDX_DIM
    out = np.empty(IDX_DIM, dtype=np.float32)
    _load().oracle_hadamard_rotate(_p(x), _p(out))
    return out


def quantize_row(xr: np.ndarray):
    """binary32 [64] -> (int8 codes [64], fp16 scale bits)."""
    xr = np.ascontiguousarray(xr, dtype=np.float32)
    assert xr.size == IDX_DIM
    codes = np.empty(IDX_DIM, dtype=np.int8)
    sc = np.zeros(1, dtype=np.uint16)
    _load().oracle_quantize_row(_p(xr), _p(codes), _p(sc))
    return codes, int(sc[0])


def c8_score(q8: np.ndarray, sq: int, k8: np.ndarray, sk: int) -> float:
    q8 = np.ascontiguousarray(q8, dtype=np.int8)
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    return float(np.float32(_load().oracle_c8_score(_p(q8), int(sq), _p(k8), int(sk))))


def f32_to_f16(x: float) -> int:
    return int(_load().oracle_f32_to_f16(float(np.float32(x))))


def f16_to_f32(h: int) -> float:
    return float(np.float32(_load().oracle_f16_to_f32(int(h))))


class LRUState:
    """One (layer, seq) residency table driven by scripted selections."""

    def __init__(self, cap: int, S: int):
        self.cap, self.S = cap, S
        self.cache_slots = np.full(cap, -1, dtype=np.int32)
        self.slot_token = np.full(S, -1, dtype=np.int32)
        self.last_use = np.full(S, -1, dtype=np.int32)
        self.t = 0

    def apply(self, selected) -> Dict[str, np.ndarray]:
        sel = np.ascontiguousarray(np.asarray(selected, dtype=np.int32))
        n = sel.size
        misses = np.empty(max(n, 1), dtype=np.int32)
        victims = np.empty(max(n, 1), dtype=np.int32)
        old = np.empty(max(n, 1), dtype=np.int32)
        nh = np.zeros(1, dtype=np.int32)
        nm = _load().oracle_lru_apply(_p(self.cache_slots), self.cap, _p(self.slot_token),
                                      _p(self.last_use), self.S, self.t, _p(sel), n,
                                      _p(misses), _p(victims), _p(old), _p(nh))
        if nm < 0:
            raise RuntimeError(f"oracle LRU failed ({nm}: -5 = not enough victims, "
                               "-7 = a residency flag disagrees with the table)")
        self.t += 1
        return {"misses": misses[:nm].copy(), "victims": victims[:nm].copy(),
                "evict_old": old[:nm].copy(), "hits": int(nh[0])}


class Oracle:
    """Whole-step oracle over [layers][batch] independent chains."""

    def __init__(self, layers: int, batch: int, capacity: int, top_k: int, hot_slots: int,
                 positions: int, heads: int, scale: float, indexer_c8: bool = False):
        self.L, self.B, self.cap = layers, batch, capacity
        self.k, self.S, self.D, self.H = top_k, hot_slots, positions, heads
        self.scale = float(np.float32(scale))
        self.c8 = bool(indexer_c8)
        self._h = _load().oracle_create(layers, batch, capacity, top_k, hot_slots,
                                         positions, heads, self.scale)
        if not self._h:
            raise ValueError("oracle_create rejected the configuration")
        if self.c8 and _load().oracle_set_indexer_c8(self._h, 1) != 0:
            raise ValueError("oracle_set_indexer_c8 failed")

    def close(self):
        if self._h:
            _load().oracle_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, layer: int, seq: int, idx_rows: np.ndarray, kv_rows: np.ndarray) -> None:
        idx_rows = np.ascontiguousarray(idx_rows, dtype=np.uint16)
        kv_rows = np.ascontiguousarray(kv_rows, dtype=np.uint16)
        n = idx_rows.shape[0]
        assert idx_rows.shape == (n, IDX_DIM) and kv_rows.shape == (n, KV_DIM)
        rc = _load().oracle_append(self._h, layer, seq, _p(idx_rows), _p(kv_rows), n)
        if rc != 0:
            raise RuntimeError(f"oracle_append failed ({rc})")

    def decode_step(self, layer: int, q_idx: np.ndarray, q_attn: np.ndarray,
                    want_keys: bool = False, want_out: bool = True,
                    want_pool_out: bool = False) -> Dict[str, np.ndarray]:
        B, D, k, H = self.B, self.D, self.k, self.H
        q_idx = np.ascontiguousarray(q_idx, dtype=np.uint16)
        q_attn = np.ascontiguousarray(q_attn, dtype=np.uint16)
        assert q_idx.shape == (B, D, IDX_DIM), q_idx.shape
        assert q_attn.shape == (B, D, H, KV_DIM), q_attn.shape
        r = {
            "topk": np.zeros((B, D, k), dtype=np.int32),
            "phys": np.zeros((B, D, k), dtype=np.int32),
            "counts": np.zeros((B, 8), dtype=np.int32),
            "misses": np.full((B, D * k), -1, dtype=np.int32),
            "victims": np.full((B, D * k), -1, dtype=np.int32),
            "evict_old": np.full((B, D * k), -1, dtype=np.int32),
        }
        keys = np.zeros((B, D, self.cap), dtype=np.uint32) if want_keys else None
        out = np.zeros((B, D, H, V_DIM), dtype=np.float64) if want_out else None
        out_pool = np.zeros((B, D, H, V_DIM), dtype=np.float64) if want_pool_out else None
        rc = _load().oracle_decode_step(self._h, layer, _p(q_idx), _p(q_attn), _p(r["topk"]),
                                        _p(r["phys"]), _p(keys), _p(r["counts"]), _p(r["misses"]),
                                        _p(r["victims"]), _p(r["evict_old"]), _p(out), _p(out_pool))
        if rc != 0:
            raise RuntimeError(f"oracle_decode_step failed ({rc})")
        if keys is not None:
            r["keys"] = keys
        if out is not None:
            r["out"] = out
        if out_pool is not None:
            r["out_pool"] = out_pool
        return r

    def indexer_c8(self, layer: int, seq: int):
        """(codes int8 [cap][64], scales fp16 bits [cap]) of one chain."""
        codes = np.empty((self.cap, IDX_DIM), dtype=np.int8)
        scales = np.empty(self.cap, dtype=np.uint16)
        if _load().oracle_read_indexer_c8(self._h, layer, seq, _p(codes), _p(scales)) != 0:
            raise RuntimeError("oracle_read_indexer_c8 failed (not in int8 mode?)")
        return codes, scales

    def state(self, layer: int, seq: int) -> Dict[str, np.ndarray]:
        cs = np.empty(self.cap, dtype=np.int32)
        st = np.empty(self.S, dtype=np.int32)
        lu = np.empty(self.S, dtype=np.int32)
        hot = np.empty((self.S, KV_DIM), dtype=np.uint16)
        nt = np.zeros(1, dtype=np.int64)
        rc = _load().oracle_read_state(self._h, layer, seq, _p(cs), _p(st), _p(lu), _p(hot), _p(nt))
        if rc != 0:
            raise RuntimeError("oracle_read_state failed")
        return {"cache_slots": cs, "slot_token": st, "last_use": lu, "hot": hot, "ntok": int(nt[0])}
