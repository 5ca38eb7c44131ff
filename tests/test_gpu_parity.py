"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Each case runs the whole step on the GPU for every sequence and compares the
oracle's chains element by element: packed winners, slots, counts, miss
lists, evictions, the residency tables and hot-buffer bytes bit-exactly;
attention within 2e-2 absolute and 1e-2 relative RMS (tests/parity_harness.py).
"""
import dataclasses
import sys

import numpy as np
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
    import sparse_kv_offload_amd  # noqa: F401  (raises if libsko.so is missing)
    yield


def case(name, **kw):
    base = dict(layers=1, batch=2, context=1500, steps=8, top_k=64, hot_slots=160, positions=1,
                heads=16, seed=4321)
    base.update(kw)
    return synth.Workload(name, **base)


def test_tiny_workload_full():
    """The tiny workload exactly as specified (1 x 1, 4096 context, 8 steps)."""
    log("case tiny")
    worst = run_parity(synth.TINY, check_keys=True, log=log)
    log(f"tiny worst {worst}")


def test_several_tiles_mtp():
    """Many score blocks, refine, several attention chunks and head groups."""
    w = case("tiles", batch=4, context=20000, steps=10, top_k=512, hot_slots=1100, positions=2,
             heads=20)
    log(f"case {w}")
    run_parity(w, check_keys=True, log=log)


@pytest.mark.parametrize("device_append", [True, False])
def test_ragged_batch(device_append):
    """Per-sequence lengths differ; one sequence is shorter than k."""
    w = case("ragged", batch=3, contexts=(3001, 1, 777), context=3001, steps=9, top_k=100,
             hot_slots=337, positions=3, heads=5)
    log(f"case ragged device_append={device_append}")
    run_parity(w, check_keys=True, device_append=device_append, log=log)


@pytest.mark.parametrize("pool", ["coherent", "noncoherent"])
def test_pool_modes(pool):
    """Both host-pool allocation modes give identical results."""
    import sparse_kv_offload_amd as sko
    flags = {"coherent": sko.SKO_FLAG_POOL_COHERENT, "noncoherent": sko.SKO_FLAG_POOL_NONCOHERENT}[pool]
    w = case("pool", batch=3, context=2500, steps=10, top_k=128, hot_slots=300, positions=2, heads=16)
    log(f"case pool={pool}")
    run_parity(w, check_keys=True, flags=flags, log=log)


def test_minimum_shelf():
    """S == D*k: every non-hit slot is a victim candidate each step."""
    w = case("minshelf", batch=2, context=900, steps=20, top_k=64, hot_slots=128, positions=2, heads=3)
    log("case minshelf")
    run_parity(w, log=log)


def test_five_positions():
    """D = 5: the score runs two position groups (4 + 1)."""
    w = case("d5", batch=2, context=1200, steps=8, top_k=40, hot_slots=230, positions=5, heads=7)
    log("case d5")
    run_parity(w, check_keys=True, log=log)


@pytest.mark.parametrize("positions", [16, 17])
def test_many_positions(positions):
    """16 positions: the largest count whose lists the LRU update puts in
    token order; 17: the lists keep the selection's order."""
    w = case(f"d{positions}", batch=2, context=1500, steps=6, top_k=24, hot_slots=positions * 24 + 40,
             positions=positions, heads=4)
    log(f"case d{positions}")
    run_parity(w, log=log)


def test_k_equals_one():
    w = case("k1", batch=2, context=700, steps=12, top_k=1, hot_slots=1, positions=1, heads=4)
    log("case k1")
    run_parity(w, check_keys=True, log=log)


@dataclasses.dataclass(frozen=True)
class TiedRows(synth.Workload):
    """Indexer rows repeat with period 7: every score occurs many times."""
    period: int = 7

    def index_rows(self, layer, seq, row0, n, out=None):
        rows = np.arange(row0, row0 + n) % self.period
        base = synth.Workload.index_rows(self, layer, seq, 0, self.period)
        return np.ascontiguousarray(base[rows])


def test_score_ties_go_to_smaller_index():
    w = TiedRows("ties", layers=1, batch=2, context=2000, steps=6, top_k=300, hot_slots=700,
                 positions=2, heads=2, seed=99)
    log("case ties")
    run_parity(w, check_keys=True, log=log)


@dataclasses.dataclass(frozen=True)
class ZeroQuery(synth.Workload):
    """All indexer queries are zero: every score is +0 and the winners are
    the k smallest token indices."""

    def index_queries(self, layer, seq, steps=None):
        T = self.steps if steps is None else steps
        return np.zeros((T, self.positions, 64), dtype=np.uint16)


def test_zero_query_all_ties():
    w = ZeroQuery("zeroq", layers=1, batch=2, context=5000, steps=4, top_k=200, hot_slots=400,
                  positions=2, heads=16, seed=5)
    log("case zero query")
    run_parity(w, check_keys=True, log=log)


def test_empty_sequence_gives_zero_output():
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=2, batch=3, max_tokens=600, num_heads=16, top_k=32,
                          hot_slots=64, mtp_positions=1)
    with sko.SparseKVOffload(cfg, torch.cuda.current_stream()) as h:
        w = case("empty", batch=3, context=500)
        h.append(1, 0, w.index_rows(1, 0, 0, 500), w.kv_rows(1, 0, 0, 500))
        qi = torch.ones((3, 1, 64), dtype=torch.int16, device="cuda") * 0x3F80  # bf16 1.0
        qa = torch.zeros((3, 1, 16, 576), dtype=torch.int16, device="cuda")
        out = torch.full((3, 1, 16, 512), 7.0, device="cuda")
        h.decode_step(1, qi, qa, out)
        torch.cuda.synchronize()
        cn = h.step_buffer(sko.SKO_BUF_COUNTS)
        assert cn[0, 4] == 32 and cn[0, 2] == 32 and cn[0, 6] == 0
        assert np.all(cn[1:, :5] == 0)
        o = out.cpu().numpy()
        assert np.all(o[1:] == 0.0)
        # q_attn = 0 -> uniform softmax -> mean of V over the 32 winners
        assert np.all(np.isfinite(o[0])) and np.abs(o[0]).max() < 2.0
        # layer 0 was never touched; its step stamp is independent
        h.decode_step(0, qi, qa, out)
        torch.cuda.synchronize()
        assert np.all(h.step_buffer(sko.SKO_BUF_COUNTS)[:, :5] == 0)
        assert np.all(out.cpu().numpy() == 0.0)


def test_early_copy_with_empty_first_sequence():
    """Early copy while sequence 0 holds no tokens (its attention blocks have
    no rows): the per-step copy state must still be reset, so over
    several steps with new misses the results equal the late copy's
    (selection and hot-buffer rows bit for bit)."""
    import torch
    import sparse_kv_offload_amd as sko
    w = case("empty0", batch=2, context=700, top_k=32)
    handles = []
    for f in (0, sko.SKO_FLAG_LATE_COPY):
        cfg = sko.make_config(num_layers=1, batch=2, max_tokens=700, num_heads=16, top_k=32,
                              hot_slots=64, mtp_positions=1, flags=f)
        handles.append(sko.SparseKVOffload(cfg, torch.cuda.current_stream()))
    try:
        for h in handles:
            h.append(0, 1, w.index_rows(0, 1, 0, 400), w.kv_rows(0, 1, 0, 400))
        gen = torch.Generator().manual_seed(11)
        for step in range(6):
            log(f"case empty0 step {step}")
            lo = 400 + 40 * step
            qi = (torch.randn((2, 1, 64), generator=gen) * 0.3).to(torch.bfloat16).view(torch.int16).cuda()
            qa = (torch.randn((2, 1, 16, 576), generator=gen) * 0.3).to(torch.bfloat16).view(torch.int16).cuda()
            outs = []
            for h in handles:
                h.append(0, 1, w.index_rows(0, 1, lo, 40), w.kv_rows(0, 1, lo, 40))
                out = torch.full((2, 1, 16, 512), 7.0, device="cuda")
                h.decode_step(0, qi, qa, out)
                torch.cuda.synchronize()
                outs.append((out.cpu().numpy(), h.step_buffer(sko.SKO_BUF_COUNTS),
                             h.step_buffer(sko.SKO_BUF_PHYS), h.table(0, 1, sko.SKO_TAB_HOT)))
            (oe, ce, pe, he), (ol, cl, pl, hl) = outs
            assert ce[1, 2] > 0, "every step must miss"
            assert np.array_equal(ce, cl) and ce[0, 4] == 0 and ce[1, 4] == 32
            assert np.array_equal(pe[1], pl[1])  # (sequence 0 selects nothing)
            # same arithmetic on the same rows; only the copy path differs
            assert np.abs(oe - ol).max() <= 1e-5, f"step {step}: outputs differ"
            assert np.all(oe[0] == 0.0)
            assert np.array_equal(he, hl), f"step {step}: hot rows differ"
    finally:
        for h in handles:
            h.close()


def test_append_capacity_and_validation_on_device():
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=1, batch=2, max_tokens=100, num_heads=1, top_k=8,
                          hot_slots=8, mtp_positions=1)
    with sko.SparseKVOffload(cfg, torch.cuda.current_stream()) as h:
        w = case("cap", batch=2, context=100, top_k=8)
        h.append(0, 1, w.index_rows(0, 1, 0, 90), w.kv_rows(0, 1, 0, 90))
        with pytest.raises(sko.SkoError) as e:
            h.append(0, sko.SKO_ALL_SEQS, np.zeros((2 * 11, 64), np.uint16), np.zeros((2 * 11, 576), np.uint16), 11)
        assert e.value.code == sko.SKO_E_CAPACITY
        # nothing was written by the rejected call
        assert h.table(0, 0, sko.SKO_TAB_NTOK)[0] == 0 and h.table(0, 1, sko.SKO_TAB_NTOK)[0] == 90
        with pytest.raises(sko.SkoError) as e:
            h.decode_step(3, 0, 0, 0)
        assert e.value.code == sko.SKO_E_INVAL
        # pool rows land where they belong
        pool = h.table(0, 1, sko.SKO_TAB_POOL)
        assert np.array_equal(pool[:90], w.kv_rows(0, 1, 0, 90))
        idx = h.table(0, 1, sko.SKO_TAB_INDEXER)
        assert np.array_equal(idx[:90], w.index_rows(0, 1, 0, 90))


@pytest.mark.parametrize("name", ["tiles", "ragged", "ties", "zeroq"])
def test_rescan_path(name):
    """The selection's rescan path (forced for every row) gives the same
    winners as the oracle."""
    import sparse_kv_offload_amd as sko
    if name == "tiles":
        w = case("tiles_rescan", batch=3, context=9000, steps=6, top_k=256, hot_slots=600, positions=2,
                 heads=4)
    elif name == "ragged":
        w = case("ragged_rescan", batch=3, contexts=(3001, 1, 777), context=3001, steps=6, top_k=100,
                 hot_slots=337, positions=3, heads=5)
    elif name == "ties":
        w = TiedRows("ties_rescan", layers=1, batch=2, context=2000, steps=4, top_k=300, hot_slots=700,
                     positions=2, heads=2, seed=99)
    else:
        w = ZeroQuery("zeroq_rescan", layers=1, batch=2, context=5000, steps=3, top_k=200, hot_slots=400,
                      positions=2, heads=16, seed=5)
    log(f"case rescan {name}")
    worst = run_parity(w, check_keys=(name != "zeroq"), flags=sko.SKO_FLAG_SELECT_RESCAN, log=log)
    log(f"rescans {worst['rescans']}")


@dataclasses.dataclass(frozen=True)
class ScaledQuery(synth.Workload):
    """Indexer queries alternate between scale 1 and 1/16 (exact in bf16):
    the score threshold drops four octaves on every other step, below the
    candidate floor set from the step before."""

    def index_queries(self, layer, seq, steps=None):
        q = synth.Workload.index_queries(self, layer, seq, steps)
        f = (q.astype(np.uint32) << 16).view(np.float32).copy()
        f[1::2] *= np.float32(1.0 / 16.0)
        return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_floor_below_threshold_rescans():
    """A threshold that falls below the floor takes the rescan path on its
    own; the results still match the oracle."""
    w = ScaledQuery("scaledq", layers=1, batch=2, context=6000, steps=6, top_k=128, hot_slots=300,
                    positions=2, heads=4, seed=17)
    log("case scaled query")
    worst = run_parity(w, check_keys=True, log=log)
    rows = w.batch * w.positions
    log(f"rescans {worst['rescans']} of {w.steps * rows} rows")
    assert rows <= worst["rescans"] < w.steps * rows


def test_keys_need_keep_flag():
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=1, batch=1, max_tokens=100, num_heads=1, top_k=8, hot_slots=8,
                          mtp_positions=1)
    with sko.SparseKVOffload(cfg, torch.cuda.current_stream()) as h:
        with pytest.raises(sko.SkoError) as e:
            h.step_buffer(sko.SKO_BUF_KEYS)
        assert e.value.code == sko.SKO_E_STATE


@pytest.mark.parametrize("mode", ["early", "fused", "late"])
def test_copy_modes_one_position(mode):
    """One position, 16 heads: the early copy (the default), the
    copy inside the attention launch and the late copy all give the oracle's
    results, hot-buffer bytes included."""
    import sparse_kv_offload_amd as sko
    w = case("copy", batch=3, context=12000, steps=8, top_k=300, hot_slots=700, positions=1, heads=16)
    log(f"case copy mode={mode}")
    f = {"early": 0, "fused": sko.SKO_FLAG_FUSED_COPY, "late": sko.SKO_FLAG_LATE_COPY}[mode]
    run_parity(w, check_keys=False, flags=f, log=log)


@pytest.mark.parametrize("mode", ["late", "early"])
def test_copy_modes_positions_and_head_groups(mode):
    """Two positions and two head groups: a missed row is read by several
    attention blocks.  Late copy, and early copy (forced by its flag): the
    blocks read the one row the copy wrote."""
    import sparse_kv_offload_amd as sko
    w = case(mode, batch=3, context=9000, steps=6, top_k=256, hot_slots=600, positions=2, heads=20)
    log(f"case {mode} D=2 H=20")
    f = {"late": sko.SKO_FLAG_LATE_COPY, "early": sko.SKO_FLAG_EARLY_COPY}[mode]
    run_parity(w, check_keys=True, flags=f, log=log)


def test_early_copy_three_positions():
    """Early copy at three positions and a larger batch."""
    w = case("early", batch=6, context=5000, steps=5, top_k=128, hot_slots=500, positions=3, heads=4)
    log("case early copy B=6 D=3")
    run_parity(w, check_keys=False, flags=0, log=log)


@pytest.mark.parametrize("shape", ["d1", "d2_hg2", "d3", "d4_ragged"])
def test_hit_overlap(shape):
    """Attention split by residency (SKO_FLAG_HIT_OVERLAP): the resident
    rows are attended on the side stream beside the copy launch, the missed
    rows after it, and the combine merges both phases.  Everything the
    oracle checks, hot-buffer bytes included, at one to four positions, two
    head groups and a ragged batch."""
    import sparse_kv_offload_amd as sko
    shapes = {
        "d1": dict(batch=3, context=12000, steps=8, top_k=300, hot_slots=700, positions=1, heads=16),
        "d2_hg2": dict(batch=3, context=9000, steps=6, top_k=256, hot_slots=600, positions=2, heads=20),
        "d3": dict(batch=6, context=5000, steps=5, top_k=128, hot_slots=500, positions=3, heads=4),
        "d4_ragged": dict(batch=5, contexts=(3000, 1, 777, 2048, 150), context=3000, steps=6, top_k=200,
                          hot_slots=900, positions=4, heads=16),
    }
    w = case("overlap_" + shape, **shapes[shape])
    log(f"case hit overlap {shape}")
    run_parity(w, check_keys=False, flags=sko.SKO_FLAG_HIT_OVERLAP, log=log)


def test_hit_overlap_newest_token():
    """The newest token at every step with the split attention (it is a miss
    at its first selection, then a hit)."""
    import sparse_kv_offload_amd as sko
    w = NewestWins("newest_overlap", layers=2, batch=3, context=3000, steps=5, top_k=128, hot_slots=300,
                   positions=2, heads=16, seed=12)
    log("case newest token, hit overlap")
    run_parity(w, check_keys=False, flags=sko.SKO_FLAG_HIT_OVERLAP, log=log)


@pytest.mark.parametrize("shape", ["d1", "d4_ragged", "host_append", "zeroq", "rescan", "floor_drop"])
def test_indexer_c8(shape):
    """The int8 indexer: codes and fp16 scales of every appended row, the
    score keys of every token, the winners and everything after them match
    the oracle in its int8 mode."""
    import sparse_kv_offload_amd as sko
    f = sko.SKO_FLAG_INDEXER_C8
    device_append = True
    if shape == "d1":
        w = case("c8d1", batch=3, context=5000, steps=6, top_k=256, hot_slots=600, positions=1, heads=16)
    elif shape == "d4_ragged":
        w = case("c8d4", batch=3, contexts=(4097, 1, 900), context=4097, steps=5, top_k=128, hot_slots=600,
                 positions=4, heads=16)
    elif shape == "host_append":
        w = case("c8host", batch=2, context=3000, steps=4, top_k=100, hot_slots=300, positions=2, heads=8)
        device_append = False
    elif shape == "zeroq":
        w = ZeroQuery("c8zeroq", layers=1, batch=2, context=3000, steps=3, top_k=150, hot_slots=400,
                      positions=2, heads=16, seed=5)
    elif shape == "rescan":
        w = case("c8rescan", batch=2, context=4000, steps=4, top_k=200, hot_slots=700, positions=3, heads=16)
        f |= sko.SKO_FLAG_SELECT_RESCAN
    else:
        w = ScaledQuery("c8scaledq", layers=1, batch=2, context=6000, steps=6, top_k=128, hot_slots=300,
                        positions=1, heads=16, seed=9)
    log(f"case indexer c8 {shape}")
    worst = run_parity(w, check_keys=True, device_append=device_append, flags=f, log=log)
    if shape == "floor_drop":
        assert worst["rescans"] > 0
    log(f"c8 {shape} worst {worst}")


class NewestWins(synth.Workload):
    """Each step's new indexer row is 4x the first position's query of that
    step, so every position selects the newest token: it is a miss at every
    step (it was never resident)."""

    def index_rows(self, layer, seq, row0, n, out=None):
        rows = synth.Workload.index_rows(self, layer, seq, row0, n).copy()
        ctx = self.seq_context(seq)
        q = self.index_queries(layer, seq)
        for r in range(max(row0, ctx), row0 + n):
            f = (q[r - ctx, 0].astype(np.uint32) << 16).view(np.float32) * np.float32(4.0)
            rows[r - row0] = (f.view(np.uint32) >> 16).astype(np.uint16)
        return rows


@pytest.mark.parametrize("mode", ["early", "late", "fused"])
def test_newest_token_row_from_device(mode):
    """The newest token is selected at every step: its row is moved into the
    hot buffer from the device copy kept by the append (no host read), with
    the oracle's results, hot-buffer bytes included."""
    import sparse_kv_offload_amd as sko
    w = NewestWins("newest", layers=2, batch=3, context=3000, steps=5, top_k=128, hot_slots=300,
                   positions=1 if mode == "fused" else 2, heads=16, seed=12)
    f = {"early": 0, "late": sko.SKO_FLAG_LATE_COPY, "fused": sko.SKO_FLAG_FUSED_COPY}[mode]
    log(f"case newest token {mode}")
    run_parity(w, check_keys=False, flags=f, log=log)
    # a second run only for the counters (parity already shown above)
    import torch
    cfg = sko.make_config(num_layers=1, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                          top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions, flags=f)
    with sko.SparseKVOffload(cfg, torch.cuda.current_stream()) as h:
        for b in range(w.batch):
            h.append(0, b, w.index_rows(0, b, 0, w.context), w.kv_rows(0, b, 0, w.context))
        qs = [w.index_queries(0, b) for b in range(w.batch)]
        for t in range(w.steps):
            idx = np.concatenate([w.index_rows(0, b, w.context + t, 1) for b in range(w.batch)])
            kv = np.concatenate([w.kv_rows(0, b, w.context + t, 1) for b in range(w.batch)])
            h.append(0, sko.SKO_ALL_SEQS, torch.from_numpy(idx.view(np.int16)).cuda(),
                     torch.from_numpy(kv.view(np.int16)).cuda(), 1)
            qi = torch.from_numpy(np.stack([qs[b][t] for b in range(w.batch)]).view(np.int16)).cuda()
            qa = torch.from_numpy(np.stack([w.attn_queries(0, b, t) for b in range(w.batch)]).view(np.int16)).cuda()
            out = torch.empty((w.batch, w.positions, w.heads, 512), device="cuda")
            h.decode_step(0, qi, qa, out)
        st = h.stats(0)
    log(f"newest {mode}: direct {st.direct_rows} misses {st.misses} h2d {st.h2d_bytes}")
    assert st.direct_rows == w.steps * w.batch
    assert st.h2d_bytes == (st.misses - st.direct_rows) * 1152
