"""The fused append and decode step (sko_decode_step_append).

* Parity with the CPU oracle through the parity harness, with each step's
  new token passed to the decode call instead of to sko_append_token: many
  tiles and positions, ragged lengths (an empty sequence, and lengths that
  put the new token at the last lane of a tile or alone in a new tile), five
  positions (two score launches), the int8 indexer and every copy mode.
* Bit-exact agreement with the two calls it replaces: two handles over the
  same inputs, one per path, give the same counts, winners and their slots
  (the kk defined entries of each position), miss, victim and evicted-owner
  lists and output bits at every step, and the same residency tables,
  device rows, indexer cache, host pool and token counts after the last
  step.
* The capacity check: a sequence at max_tokens is refused before any work.
"""
import numpy as np
import pytest

import synth
from parity_harness import GpuSide, Inputs, run_parity

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
                heads=16, seed=8765)
    base.update(kw)
    return synth.Workload(name, **base)


CASES = {
    "tiles": dict(batch=4, context=20000, steps=10, top_k=512, hot_slots=1100, positions=2, heads=20),
    # the new token at lane 0 of a fresh tile (64), at lane 63 (127), in an
    # empty sequence (0), and in a long one
    "edges": dict(batch=5, contexts=(0, 63, 64, 127, 1000), context=1000, steps=70, top_k=64,
                  hot_slots=160, positions=1, heads=3),
    "five_positions": dict(batch=2, context=3000, steps=8, top_k=100, hot_slots=600, positions=5, heads=16),
    "mtp3": dict(layers=2, batch=3, context=6000, steps=8, top_k=256, hot_slots=1300, positions=4, heads=16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_append_oracle_parity(name):
    w = case("fa_" + name, **CASES[name])
    log(f"case {w}")
    run_parity(w, check_keys=True, fused_append=True, log=log)


@pytest.mark.parametrize("flag", ["INDEXER_C8", "LATE_COPY", "FUSED_COPY", "HIT_OVERLAP", "SELECT_RESCAN"])
def test_fused_append_oracle_parity_modes(flag):
    import sparse_kv_offload_amd as sko
    f = getattr(sko, "SKO_FLAG_" + flag)
    kw = dict(batch=3, context=5000, steps=8, top_k=128, hot_slots=400, positions=1, heads=16)
    if flag in ("INDEXER_C8", "SELECT_RESCAN"):
        kw.update(positions=4, hot_slots=1000)
    w = case("fa_" + flag.lower(), **kw)
    log(f"case {w} flag {flag}")
    run_parity(w, check_keys=flag != "HIT_OVERLAP", fused_append=True, flags=f, log=log)


@pytest.mark.parametrize("flags_name", ["default", "INDEXER_C8", "LATE_COPY", "FUSED_COPY"])
def test_fused_append_matches_two_calls(flags_name):
    import sparse_kv_offload_amd as sko
    flags = 0 if flags_name == "default" else getattr(sko, "SKO_FLAG_" + flags_name)
    positions = 1 if flags_name == "FUSED_COPY" else 5
    w = case("fa_exact", layers=2, batch=3, contexts=(2000, 63, 700), context=2000, steps=12, top_k=96,
             hot_slots=96 * positions + 200, positions=positions, heads=16)
    log(f"case {w} flags {flags_name}")
    L, T = w.layers, w.steps
    inputs = Inputs(w, list(range(L)), T)
    two = GpuSide(w, L, flags=flags)
    one = GpuSide(w, L, flags=flags, fused_append=True)
    seqs = list(range(w.batch))
    try:
        for side in (two, one):
            for l in range(L):
                for b in seqs:
                    side.load_prefix(l, b)
        for t in range(T):
            for l in range(L):
                qi, qa = inputs.q_idx_step(l, t, seqs), inputs.q_attn_step(l, t, seqs)
                res = []
                for side in (two, one):
                    side.append_token(l, t)
                    res.append(side.decode(l, qi, qa))
                a, b_ = res
                where = f"t={t} layer={l}"
                # the defined entries: the whole counts record, each
                # position's kk winners and their slots (both in token order),
                # the nM misses, victims and evicted owners, every output bit
                assert np.array_equal(a.counts, b_.counts), f"counts differ at {where}"
                assert np.array_equal(a.out.view(np.uint32), b_.out.view(np.uint32)), f"out differs at {where}"
                for b in seqs:
                    kk, nM = int(a.counts[b][4]), int(a.counts[b][2])
                    for name in ("topk", "phys"):
                        assert np.array_equal(getattr(a, name)[b, :, :kk], getattr(b_, name)[b, :, :kk]), \
                            f"{name} differs at {where} seq={b}"
                    for name in ("misses", "victims", "evict_old"):
                        assert np.array_equal(getattr(a, name)[b, :nM], getattr(b_, name)[b, :nM]), \
                            f"{name} differs at {where} seq={b}"
        for l in range(L):
            for b in seqs:
                ta, tb = two.tables(l, b), one.tables(l, b)
                for key in ta:
                    assert np.array_equal(ta[key], tb[key]), f"table {key} differs (layer {l} seq {b})"
                for tab in (sko.SKO_TAB_INDEXER, sko.SKO_TAB_POOL, sko.SKO_TAB_NTOK):
                    x, y = two.h.table(l, b, tab), one.h.table(l, b, tab)
                    assert np.array_equal(x, y), f"table {tab} differs (layer {l} seq {b})"
                assert int(one.h.table(l, b, sko.SKO_TAB_NTOK)[0]) == w.seq_context(b) + T
        log(f"{flags_name}: {T} steps x {L} layers identical")
    finally:
        two.close()
        one.close()


def test_fused_append_refuses_a_full_sequence():
    import sparse_kv_offload_amd as sko
    torch = pytest.importorskip("torch")
    w = case("fa_full", batch=2, context=300, steps=1, top_k=32, hot_slots=64)
    side = GpuSide(w, 1)  # capacity = context + 1
    try:
        for b in range(w.batch):
            side.load_prefix(0, b)
        inputs = Inputs(w, [0], 2)
        idx = torch.zeros((w.batch, synth.INDEX_DIM), dtype=torch.int16, device="cuda")
        kv = torch.zeros((w.batch, synth.KV_DIM), dtype=torch.int16, device="cuda")
        out = torch.empty((w.batch, 1, w.heads, synth.V_DIM), dtype=torch.float32, device="cuda")
        qi = torch.from_numpy(inputs.q_idx_step(0, 0, [0, 1]).view(np.int16)).cuda()
        qa = torch.from_numpy(inputs.q_attn_step(0, 0, [0, 1]).view(np.int16)).cuda()
        side.h.decode_step_append(0, idx, kv, qi, qa, out)
        torch.cuda.synchronize()
        with pytest.raises(sko.SkoError) as e:
            side.h.decode_step_append(0, idx, kv, qi, qa, out)
        assert e.value.code == sko.SKO_E_CAPACITY
        assert int(side.h.table(0, 0, sko.SKO_TAB_NTOK)[0]) == 301
    finally:
        side.close()
