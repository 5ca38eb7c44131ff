"""The handle's stream and instrumentation calls on the GPU: decoding on a
non-default stream, and switching streams with sko_set_stream, gives the
same residency, hot-buffer bytes, counts and attention bits as the default
stream (the LRU update puts each position's winners in token order, so the
attention's split over rows, and its rounding, does not follow the order of
the selection's atomic appends); the per-stage timing counts one launch per
layer-step for each stage of the copy arrangement; the step counters follow
the calls."""
import numpy as np
import pytest

import synth

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


W = synth.Workload("api", layers=2, batch=3, context=4000, steps=5, top_k=128, hot_slots=300, positions=2,
                   heads=16, seed=77)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def run(stream_plan, flags=0, w=W):
    """Decode w on a fresh handle; stream_plan(step) gives the stream for
    that step (None: the default stream).  Returns the outputs and tables."""
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=w.layers, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                          top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions, flags=flags)
    first = stream_plan(0)
    outs, tabs, counts, tops = [], [], [], []
    with sko.SparseKVOffload(cfg, first) as h:
        for l in range(w.layers):
            for b in range(w.batch):
                h.append(l, b, w.index_rows(l, b, 0, w.context), w.kv_rows(l, b, 0, w.context))
        torch.cuda.synchronize()
        qch = {(l, b): w.index_queries(l, b, w.steps) for l in range(w.layers) for b in range(w.batch)}
        for t in range(w.steps):
            st = stream_plan(t)
            sko.sko_set_stream(h.handle, st)
            ctx = torch.cuda.stream(st) if st is not None else torch.cuda.stream(torch.cuda.current_stream())
            with ctx:
                for l in range(w.layers):
                    ni = dev(np.concatenate([w.index_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                    nk = dev(np.concatenate([w.kv_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                    qi = dev(np.stack([qch[(l, b)][t] for b in range(w.batch)]))
                    qa = dev(np.stack([w.attn_queries(l, b, t) for b in range(w.batch)]))
                    out = torch.empty((w.batch, w.positions, w.heads, synth.V_DIM), dtype=torch.float32,
                                      device="cuda")
                    sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, ni, nk, 1, True)
                    sko.sko_decode_step(h.handle, l, qi, qa, out)
                    torch.cuda.synchronize()
                    outs.append(out.cpu().numpy())
                    counts.append(h.step_buffer(sko.SKO_BUF_COUNTS).copy())
                    tops.append(h.step_buffer(sko.SKO_BUF_TOPK).copy())
        for l in range(w.layers):
            for b in range(w.batch):
                tabs.append(h.table(l, b, sko.SKO_TAB_CACHE_SLOTS).copy())
                tabs.append(h.table(l, b, sko.SKO_TAB_HOT).copy())
        steps = [h.stats(l).steps for l in range(w.layers)]
    return outs, tabs, counts, steps, tops


@pytest.mark.parametrize("flags_name", ["early", "late"])
def test_streams_give_the_same_results(flags_name):
    import torch
    import sparse_kv_offload_amd as sko
    flags = {"early": 0, "late": sko.SKO_FLAG_LATE_COPY}[flags_name]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    log(f"streams {flags_name}: default stream")
    ref = run(lambda t: None, flags)
    log(f"streams {flags_name}: one side stream")
    one = run(lambda t: s1, flags)
    log(f"streams {flags_name}: switching streams every step")
    alt = run(lambda t: s1 if t % 2 == 0 else s2, flags)
    for other in (one, alt):
        # residency tables, hot-buffer bytes and per-step counts: exact
        for a, b in zip(ref[1], other[1]):
            assert np.array_equal(a, b)
        for a, b in zip(ref[2], other[2]):
            assert np.array_equal(a, b)
        # attention: the winners are in token order, so the same bits
        for a, b in zip(ref[0], other[0]):
            assert np.array_equal(a, b), float(np.abs(a - b).max())
    assert ref[3] == [W.steps] * W.layers == one[3] == alt[3]
    # two positions: each position's list in token order, the same on every stream
    for top, t1, t2 in zip(ref[4], one[4], alt[4]):
        assert np.array_equal(top, t1) and np.array_equal(top, t2)
        tok = (top & 0x7FFFFFFF).astype(np.int64)
        assert (np.diff(tok, axis=-1) > 0).all()


W1 = synth.Workload("api1", layers=2, batch=3, context=3000, steps=4, top_k=128, hot_slots=200, positions=1,
                    heads=16, seed=78)


@pytest.mark.parametrize("flags_name", ["early", "late", "fused"])
def test_attention_is_reproducible(flags_name):
    """Two handles decoding the same inputs give the same bits, in every copy
    arrangement (one MTP position, so the fused copy applies too)."""
    import sparse_kv_offload_amd as sko
    flags = {"early": 0, "late": sko.SKO_FLAG_LATE_COPY, "fused": sko.SKO_FLAG_FUSED_COPY}[flags_name]
    log(f"reproducible {flags_name}: first run")
    a = run(lambda t: None, flags, W1)
    log(f"reproducible {flags_name}: second run")
    b = run(lambda t: None, flags, W1)
    for x, y in zip(a[0], b[0]):
        assert np.array_equal(x, y), float(np.abs(x - y).max())
    for x, y in zip(a[1] + a[2] + a[4], b[1] + b[2] + b[4]):
        assert np.array_equal(x, y)
    # each position's winners are in token order (the residency bit aside)
    for top in a[4]:
        tok = (top.reshape(W1.batch, W1.positions, W1.top_k) & 0x7FFFFFFF).astype(np.int64)
        assert (np.diff(tok, axis=-1) > 0).all()


def test_timing_counts_one_launch_per_layer_step():
    import torch
    import sparse_kv_offload_amd as sko
    w = W
    cfg = sko.make_config(num_layers=w.layers, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                          top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions)
    with sko.SparseKVOffload(cfg, torch.cuda.current_stream()) as h:
        for l in range(w.layers):
            for b in range(w.batch):
                h.append(l, b, w.index_rows(l, b, 0, w.context), w.kv_rows(l, b, 0, w.context))
        h.set_timing((1 << sko.sko_num_stages()) - 1)
        qch = {(l, b): w.index_queries(l, b, w.steps) for l in range(w.layers) for b in range(w.batch)}
        out = torch.empty((w.batch, w.positions, w.heads, synth.V_DIM), dtype=torch.float32, device="cuda")
        n = 3
        for t in range(n):
            for l in range(w.layers):
                ni = dev(np.concatenate([w.index_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                nk = dev(np.concatenate([w.kv_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                qi = dev(np.stack([qch[(l, b)][t] for b in range(w.batch)]))
                qa = dev(np.stack([w.attn_queries(l, b, t) for b in range(w.batch)]))
                sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, ni, nk, 1, True)
                h.decode_step(l, qi, qa, out)
        tm = h.timing()
        log(f"timing: {tm}")
        layer_steps = n * w.layers
        # the early copy's stages, one launch each per layer-step
        for stage in ("append_rows", "score_hist", "topk_filter", "topk_refine", "merge_lru", "attn_partial",
                      "attn_combine"):
            ms, launches = tm[stage]
            assert launches == layer_steps, (stage, launches)
            assert ms > 0.0
        assert tm.get("gather_misses", (0.0, 0))[1] == 0  # no late gather in this mode
        # block stamps of the timed LRU-update launches: a copy span and a
        # merge span per launch, their overlap no longer than either
        ov = h.copy_overlap()
        log(f"copy overlap: {ov}")
        assert ov["launches"] == layer_steps
        assert ov["copy_ms"] > 0.0 and ov["merge_ms"] > 0.0
        assert 0.0 <= ov["overlap_ms"] <= min(ov["copy_ms"], ov["merge_ms"]) + 1e-9
        # the same launches' copy spans, one per launch, on the device clock:
        # ordered within each span, and summing to the copy time above
        spans, khz = h.copy_spans()
        assert spans.shape == (layer_steps, 2) and khz > 0
        assert (spans[:, 1] > spans[:, 0]).all()
        assert abs(float((spans[:, 1] - spans[:, 0]).sum()) / khz - ov["copy_ms"]) <= 1e-6 * ov["copy_ms"] + 1e-9
        # clearing the mask clears the totals
        h.set_timing(0)
        assert all(c == 0 for _, c in h.timing().values())
        assert h.copy_overlap()["launches"] == 0
        assert h.copy_spans()[0].shape == (0, 2)
        assert [h.stats(l).steps for l in range(w.layers)] == [n] * w.layers


def run_unsynced(stream_plan, flags=0, w=W):
    """Decode w with every input and output buffer prepared up front and no
    host synchronization between calls: stream_plan(t, l) gives the stream
    for layer l at step t, set by sko_set_stream, which alone orders the
    handle's work across the switch.  Returns every step's output and the
    final tables, counts and step counters."""
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=w.layers, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                          top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions, flags=flags)
    qch = {(l, b): w.index_queries(l, b, w.steps) for l in range(w.layers) for b in range(w.batch)}
    ins = [[(dev(np.concatenate([w.index_rows(l, b, w.context + t, 1) for b in range(w.batch)])),
             dev(np.concatenate([w.kv_rows(l, b, w.context + t, 1) for b in range(w.batch)])),
             dev(np.stack([qch[(l, b)][t] for b in range(w.batch)])),
             dev(np.stack([w.attn_queries(l, b, t) for b in range(w.batch)])))
            for l in range(w.layers)] for t in range(w.steps)]
    outs = [[torch.zeros((w.batch, w.positions, w.heads, synth.V_DIM), dtype=torch.float32, device="cuda")
             for _ in range(w.layers)] for _ in range(w.steps)]
    torch.cuda.synchronize()
    with sko.SparseKVOffload(cfg, None) as h:
        for l in range(w.layers):
            for b in range(w.batch):
                h.append(l, b, w.index_rows(l, b, 0, w.context), w.kv_rows(l, b, 0, w.context))
        for t in range(w.steps):
            for l in range(w.layers):
                sko.sko_set_stream(h.handle, stream_plan(t, l))
                ni, nk, qi, qa = ins[t][l]
                sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, ni, nk, 1, True)
                sko.sko_decode_step(h.handle, l, qi, qa, outs[t][l])
        # the read calls synchronize only the last stream
        tabs = [h.table(l, b, which).copy() for l in range(w.layers) for b in range(w.batch)
                for which in (sko.SKO_TAB_CACHE_SLOTS, sko.SKO_TAB_SLOT_TOKEN, sko.SKO_TAB_LAST_USE,
                              sko.SKO_TAB_HOT)]
        counts = h.step_buffer(sko.SKO_BUF_COUNTS).copy()
        steps = [h.stats(l).steps for l in range(w.layers)]
        torch.cuda.synchronize()
        res = [o.cpu().numpy() for row in outs for o in row]
    return res, tabs, counts, steps


@pytest.mark.parametrize("flags_name", ["early", "late", "hit_overlap"])
def test_stream_switch_without_host_sync(flags_name):
    """Switching streams at every layer-step with no host synchronization
    gives the default stream's output bits, tables and counts."""
    import torch
    import sparse_kv_offload_amd as sko
    flags = {"early": 0, "late": sko.SKO_FLAG_LATE_COPY, "hit_overlap": sko.SKO_FLAG_HIT_OVERLAP}[flags_name]
    streams = [torch.cuda.Stream() for _ in range(3)]
    log(f"unsynced {flags_name}: default stream")
    ref = run_unsynced(lambda t, l: None, flags)
    log(f"unsynced {flags_name}: a new stream at every layer-step")
    alt = run_unsynced(lambda t, l: streams[(t * W.layers + l) % 3], flags)
    for a, b in zip(ref[1], alt[1]):
        assert np.array_equal(a, b)
    assert np.array_equal(ref[2], alt[2])
    assert ref[3] == alt[3] == [W.steps] * W.layers
    for a, b in zip(ref[0], alt[0]):
        if flags_name == "hit_overlap":  # list order varies with the split attention: rounding only
            assert np.abs(a - b).max() <= 2e-3
        else:
            assert np.array_equal(a, b), float(np.abs(a - b).max())


def test_broken_invariant_fails_the_handle():
    """A residency invariant the merge kernel finds broken is counted on the
    device and makes the next synchronizing read mark the handle FAILED
    (forced here by the test switch, which leaves every kernel's work
    unchanged)."""
    import torch
    import sparse_kv_offload_amd as sko
    w = W1
    for flags, broken in ((0, False), (sko.SKO_FLAG_TEST_VIOLATION, True)):
        cfg = sko.make_config(num_layers=1, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                              top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions, flags=flags)
        with sko.SparseKVOffload(cfg, None) as h:
            for b in range(w.batch):
                h.append(0, b, w.index_rows(0, b, 0, w.context + 1), w.kv_rows(0, b, 0, w.context + 1))
            qi = dev(np.stack([w.index_queries(0, b)[0] for b in range(w.batch)]))
            qa = dev(np.stack([w.attn_queries(0, b, 0) for b in range(w.batch)]))
            out = torch.zeros((w.batch, w.positions, w.heads, synth.V_DIM), dtype=torch.float32, device="cuda")
            h.decode_step(0, qi, qa, out)
            if not broken:
                assert h.stats(0).steps == 1
                continue
            with pytest.raises(sko.SkoError) as e:
                h.stats(0)
            assert e.value.code == sko.SKO_E_STATE and "invariant" in str(e.value)
            # the handle stays FAILED for every later call
            with pytest.raises(sko.SkoError) as e:
                h.decode_step(0, qi, qa, out)
            assert e.value.code == sko.SKO_E_STATE
            with pytest.raises(sko.SkoError):
                h.step_buffer(sko.SKO_BUF_COUNTS)
        torch.cuda.synchronize()
