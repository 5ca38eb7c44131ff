"""The step kept off the copy blocks' XCD (SKO_FLAG_XCD_SPLIT), alone and as
micro-batches: the batch split into handles on their own streams whose steps
overlap on the device.

Every case checks the oracle's chains element by element (packed winners,
slots, counts, miss lists, evictions, residency tables and hot-buffer bytes
bit-exactly; attention within 2e-2 absolute and 1e-2 relative RMS).  The
split changes only where blocks run: the copy blocks on one XCD, every other
block on the other seven.  The grids cover a launch smaller than one group of
eight blocks, launches that are not multiples of seven work blocks, several
score blocks per sequence, head groups, up to 17 positions, a ragged batch
with an empty sequence, and the full shelf_ctx8, small, mtp3 and long shapes
in the benchmark's micro-batch configuration (two handles).
"""
import pytest

import synth
from parity_harness import run_parity, run_parity_micro

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_kv_offload_amd as sko  # raises if libsko.so is missing
    cfg = sko.make_config(num_layers=1, batch=1, max_tokens=64, num_heads=1, top_k=4, hot_slots=8,
                          flags=sko.SKO_FLAG_XCD_SPLIT)
    try:
        sko.SparseKVOffload(cfg, None).close()
    except sko.SkoError as e:
        if e.code == sko.SKO_E_UNSUPPORTED:
            pytest.skip(f"the device does not deal launch blocks to 8 XCDs in a fixed stripe: {e}")
        raise
    yield


def case(name, **kw):
    base = dict(layers=1, batch=2, context=1500, steps=8, top_k=64, hot_slots=160, positions=1,
                heads=16, seed=4321)
    base.update(kw)
    return synth.Workload(name, **base)


@pytest.mark.parametrize("shape", ["tiny", "tiles_d2_hg2", "ragged_d3", "d5"])
@pytest.mark.parametrize("fused_append", [False, True])
def test_split_one_handle(shape, fused_append):
    """One handle with the split: the oracle's results, score keys included."""
    import sparse_kv_offload_amd as sko
    shapes = {
        "tiny": dict(batch=1, context=700, steps=6, top_k=32, hot_slots=96, positions=1, heads=16),
        "tiles_d2_hg2": dict(batch=4, context=20000, steps=6, top_k=512, hot_slots=1100, positions=2,
                             heads=20),
        "ragged_d3": dict(batch=3, contexts=(3001, 0, 777), context=3001, steps=7, top_k=100,
                          hot_slots=337, positions=3, heads=5),
        "d5": dict(batch=2, context=9000, steps=5, top_k=200, hot_slots=1000, positions=5, heads=16),
    }
    w = case(f"xcd_{shape}", **shapes[shape])
    log(f"case xcd split one handle {shape} fused_append={fused_append}: {w}")
    worst = run_parity(w, check_keys=True, flags=sko.SKO_FLAG_XCD_SPLIT, fused_append=fused_append, log=log)
    log(f"worst {worst}")


@pytest.mark.parametrize("extra", ["c8", "rescan"])
def test_split_one_handle_int8_and_rescan(extra):
    """The split with the int8 indexer (its codes and scales bit-exact) and
    with every row selected through the filter's rescan path."""
    import sparse_kv_offload_amd as sko
    w = case(f"xcd_{extra}", batch=3, context=9000, steps=5, top_k=256, hot_slots=1100, positions=4, heads=16)
    f = sko.SKO_FLAG_XCD_SPLIT | {"c8": sko.SKO_FLAG_INDEXER_C8, "rescan": sko.SKO_FLAG_SELECT_RESCAN}[extra]
    log(f"case xcd split + {extra}: {w}")
    worst = run_parity(w, check_keys=True, flags=f, fused_append=True, log=log)
    log(f"worst {worst}")


@pytest.mark.parametrize("positions", [16, 17])
def test_split_many_positions(positions):
    """The split with four and five score launches per step (16 and 17
    positions, four positions per launch) and the LRU update over D * k
    entries: 16 is the largest count whose lists the LRU update puts in
    token order, with 17 the lists keep the selection's order."""
    import sparse_kv_offload_amd as sko
    w = case(f"xcd_d{positions}", batch=3, context=1500, steps=6, top_k=24, hot_slots=positions * 24 + 40,
             positions=positions, heads=4)
    log(f"case xcd split d{positions}: {w}")
    worst = run_parity(w, check_keys=True, flags=sko.SKO_FLAG_XCD_SPLIT, fused_append=True, log=log)
    log(f"worst {worst}")


@pytest.mark.parametrize("shape,nmb", [("d1", 2), ("d4", 2), ("ragged_d2", 3), ("d5", 2)])
def test_micro_batches_each_layer(shape, nmb):
    """nmb handles on nmb streams, every layer's calls of all handles queued
    before one wait: each handle's results against the oracle at every step."""
    shapes = {
        "d1": dict(batch=4, context=12000, steps=8, top_k=300, hot_slots=700, positions=1, heads=16),
        "d4": dict(batch=4, layers=2, context=9000, steps=6, top_k=256, hot_slots=1100, positions=4,
                   heads=16),
        "ragged_d2": dict(batch=5, contexts=(2000, 0, 4100, 63, 64), context=4100, steps=6, top_k=64,
                          hot_slots=200, positions=2, heads=20),
        # two score launches per step in each handle
        "d5": dict(batch=4, context=6000, steps=6, top_k=128, hot_slots=900, positions=5, heads=16),
    }
    w = case(f"micro_{shape}", **shapes[shape])
    log(f"case micro-batches {nmb} {shape}: {w}")
    worst = run_parity_micro(w, nmb=nmb, log=log)
    log(f"worst {worst}")


def test_micro_batches_queued_without_waits():
    """Two handles, two layers, the whole run queued with no wait between
    steps (layer l + 1 of one handle overlaps layer l of the other): the last
    step and every table at the end against the oracle."""
    w = case("micro_async", batch=4, layers=2, context=8000, steps=10, top_k=256, hot_slots=600,
             positions=2, heads=16)
    log(f"case micro-batches queued: {w}")
    worst = run_parity_micro(w, nmb=2, sync_each_layer=False, log=log)
    log(f"worst {worst}")


def test_micro_batches_shelf_ctx8_full_shape():
    """shelf_ctx8 at full shape (B = 32 in two handles of 16, 64K context,
    k 2048, S 8192) in the benchmark's launch configuration: one layer, 24
    steps, one chain in each handle."""
    w = synth.SHELF8
    log(f"fullsize shelf_ctx8 micro-batches 2: {w}")
    worst = run_parity_micro(w, nmb=2, layers=1, steps=24, chains=[(0, 3), (0, 30)],
                             out_steps={0, 1, 12, 23}, check_tables_every=8, log=log)
    log(f"worst {worst}")


def test_micro_batches_small_full_shape():
    """small at full shape (B = 8 in two handles of 4, 32K context, k 2048,
    S 4096, 4 layers), the benchmark's default for it: 12 steps, a chain in
    each handle on different layers."""
    w = synth.SMALL
    log(f"fullsize small micro-batches 2: {w}")
    worst = run_parity_micro(w, nmb=2, layers=4, steps=12, chains=[(0, 1), (3, 6)],
                             out_steps={0, 1, 11}, check_tables_every=4, log=log)
    log(f"worst {worst}")


def test_micro_batches_mtp3_full_shape():
    """mtp3 at full shape (B = 16 in two handles of 8, 128K context, four
    positions, k 2048, S 16384), the benchmark's default for it: one layer,
    12 steps, a chain in each handle."""
    w = synth.MTP3
    log(f"fullsize mtp3 micro-batches 2: {w}")
    worst = run_parity_micro(w, nmb=2, layers=1, steps=12, chains=[(0, 2), (0, 13)],
                             out_steps={0, 1, 11}, check_tables_every=4, log=log)
    log(f"worst {worst}")


def test_micro_batches_long_full_shape():
    """long at full shape (B = 2 in two handles of one sequence, 1M-token
    context, four positions, k 2048, S 131072), the benchmark's default for
    it: one layer, 8 steps, both chains."""
    w = synth.LONG
    log(f"fullsize long micro-batches 2: {w}")
    worst = run_parity_micro(w, nmb=2, layers=1, steps=8, chains=[(0, 0), (0, 1)],
                             out_steps={0, 1, 7}, check_tables_every=4, log=log)
    log(f"worst {worst}")
