"""Parity at the full workload sizes, in the benchmark's launch configuration.

The GPU runs every sequence of the workload at its real per-layer shape (the
same kernels and grids the benchmark times); the oracle replays sampled
(layer, seq) chains one by one (chains are independent, so a chain replayed
alone is the full workload restricted to it).  Every step is compared
bit-exactly on selection, counts, misses and evictions; attention is checked
on a few steps; residency tables and hot-buffer bytes every few steps.

Long horizons are covered: shelf_ctx8 runs one chain through all 256 steps
(topic jumps at 64, 128 and 192, so the ring compaction and the candidate
floor are exercised after each jump), mtp3 runs all 4 layers for 64 steps
with two chains, long runs all 64 steps.  The GPU runs 2 of shelf's 8
layers (the other layers repeat identical launches on more memory).
"""
import pytest

import synth
from parity_harness import run_parity

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_kv_offload_amd  # noqa: F401
    yield


def _run(w, layers, steps, chains, out_steps, tables_every, flags=0):
    log(f"fullsize {w.name}: layers={layers} batch={w.batch} context={w.context} k={w.top_k} "
        f"S={w.hot_slots} D={w.positions} H={w.heads} steps={steps} chains={chains} flags={flags:#x}")
    worst = run_parity(w, layers=layers, steps=steps, chains=chains, out_steps=set(out_steps),
                       check_tables_every=tables_every, log=log, flags=flags)
    log(f"fullsize {w.name}: ok, attention worst {worst}")


def test_small_full():
    w = synth.SMALL
    _run(w, layers=4, steps=w.steps, chains=[(0, 0), (3, 7)], out_steps=[0, 1, 31, 63],
         tables_every=16)


def test_mtp3_full_all_layers():
    w = synth.MTP3
    _run(w, layers=4, steps=64, chains=[(0, 3), (3, 15)], out_steps=range(0, 64, 16), tables_every=16)


def test_shelf_ctx8_all_steps_across_topic_jumps():
    w = synth.SHELF8
    _run(w, layers=2, steps=w.steps, chains=[(1, 31)], out_steps=list(range(0, 256, 32)) + [255],
         tables_every=32)


def test_shelf_ctx4_full_shape():
    w = synth.SHELF4
    _run(w, layers=1, steps=70, chains=[(0, 5)], out_steps=[0, 64, 69], tables_every=32)


def test_long_all_steps():
    w = synth.LONG
    _run(w, layers=2, steps=w.steps, chains=[(1, 1)], out_steps=list(range(0, 64, 16)) + [63],
         tables_every=16)


def test_long_full_shape_int8_indexer():
    """The int8 indexer at the long workload's shape (codes, scales and
    tables of the sampled chain compared too)."""
    import sparse_kv_offload_amd as sko
    w = synth.LONG
    _run(w, layers=1, steps=6, chains=[(0, 1)], out_steps=[0, 5], tables_every=5,
         flags=sko.SKO_FLAG_INDEXER_C8)


def test_mtp3_full_shape_int8_indexer():
    import sparse_kv_offload_amd as sko
    w = synth.MTP3
    _run(w, layers=1, steps=8, chains=[(0, 9)], out_steps=[0, 7], tables_every=7,
         flags=sko.SKO_FLAG_INDEXER_C8)


def test_mtp3_full_shape_hit_overlap():
    """The split attention at the mtp3 shape (four positions, 16 sequences)."""
    import sparse_kv_offload_amd as sko
    w = synth.MTP3
    _run(w, layers=1, steps=10, chains=[(0, 6)], out_steps=[0, 9], tables_every=9,
         flags=sko.SKO_FLAG_HIT_OVERLAP)


def test_small_full_hit_overlap():
    import sparse_kv_offload_amd as sko
    w = synth.SMALL
    _run(w, layers=2, steps=24, chains=[(1, 5)], out_steps=[0, 23], tables_every=12,
         flags=sko.SKO_FLAG_HIT_OVERLAP)
