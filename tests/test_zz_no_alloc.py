"""The decode step without allocation (sko_decode_step_static) against the
ordinary entry point: the same kernels with their per-step scratch taken
from the library's static device array.  Two workloads in a row, the second
smaller, so the array holds the first one's leftovers when the second
starts; every step's output bits, counts and lists and the final tables
must equal those of a handle driven by sko_decode_step on the same inputs."""
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


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def handle(sko, w, flags=0):
    cfg = sko.make_config(num_layers=w.layers, batch=w.batch, max_tokens=w.capacity, num_heads=w.heads,
                          top_k=w.top_k, hot_slots=w.hot_slots, mtp_positions=w.positions, flags=flags)
    h = sko.SparseKVOffload(cfg, None)
    for l in range(w.layers):
        for b in range(w.batch):
            h.append(l, b, w.index_rows(l, b, 0, w.context), w.kv_rows(l, b, 0, w.context))
    return h


def compare_workload(w, flags=0):
    import torch
    import sparse_kv_offload_amd as sko
    ref, nz = handle(sko, w, flags), handle(sko, w, flags)
    qch = {(l, b): w.index_queries(l, b, w.steps) for l in range(w.layers) for b in range(w.batch)}
    try:
        for t in range(w.steps):
            for l in range(w.layers):
                ni = dev(np.concatenate([w.index_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                nk = dev(np.concatenate([w.kv_rows(l, b, w.context + t, 1) for b in range(w.batch)]))
                qi = dev(np.stack([qch[(l, b)][t] for b in range(w.batch)]))
                qa = dev(np.stack([w.attn_queries(l, b, t) for b in range(w.batch)]))
                outs = []
                for h, step in ((ref, sko.sko_decode_step), (nz, sko.sko_decode_step_static)):
                    out = torch.full((w.batch, w.positions, w.heads, synth.V_DIM), float("nan"),
                                     dtype=torch.float32, device="cuda")
                    sko.sko_append_token(h.handle, l, sko.SKO_ALL_SEQS, ni, nk, 1, True)
                    step(h.handle, l, qi, qa, out)
                    torch.cuda.synchronize()
                    outs.append((out.cpu().numpy(), [h.step_buffer(x).copy() for x in
                                                     (sko.SKO_BUF_TOPK, sko.SKO_BUF_PHYS, sko.SKO_BUF_COUNTS,
                                                      sko.SKO_BUF_MISSES, sko.SKO_BUF_VICTIMS,
                                                      sko.SKO_BUF_EVICT_OLD)]))
                (o_ref, b_ref), (o_nz, b_nz) = outs
                assert np.isfinite(o_ref).all()
                assert np.array_equal(o_ref, o_nz), (w.name, t, l, float(np.nanmax(np.abs(o_ref - o_nz))))
                # counts in full; the lists up to their valid lengths (the
                # rest of each buffer is undefined)
                top_r, phys_r, cnt_r, *lists_r = b_ref
                top_n, phys_n, cnt_n, *lists_n = b_nz
                assert np.array_equal(cnt_r, cnt_n), (w.name, t, l)
                cnt = cnt_r.reshape(w.batch, 8)
                for b in range(w.batch):
                    sel, nm = int(cnt[b, 4]), int(cnt[b, 2])
                    for x, y in ((top_r, top_n), (phys_r, phys_n)):
                        xb = x.reshape(w.batch, w.positions, w.top_k)[b, :, :sel]
                        yb = y.reshape(w.batch, w.positions, w.top_k)[b, :, :sel]
                        assert np.array_equal(xb, yb), (w.name, t, l, b)
                    for x, y in zip(lists_r, lists_n):
                        assert np.array_equal(x.reshape(w.batch, -1)[b, :nm], y.reshape(w.batch, -1)[b, :nm]), \
                            (w.name, t, l, b)
        for l in range(w.layers):
            for b in range(w.batch):
                for which in (sko.SKO_TAB_CACHE_SLOTS, sko.SKO_TAB_SLOT_TOKEN, sko.SKO_TAB_LAST_USE,
                              sko.SKO_TAB_HOT):
                    assert np.array_equal(ref.table(l, b, which), nz.table(l, b, which)), (w.name, l, b, which)
            assert ref.stats(l).misses == nz.stats(l).misses
    finally:
        ref.close()
        nz.close()


BIG = synth.Workload("noalloc_big", layers=2, batch=4, context=9000, steps=3, top_k=256, hot_slots=600,
                     positions=2, heads=16, seed=501)
SMALL = synth.Workload("noalloc_small", layers=1, batch=2, context=3000, steps=2, top_k=128, hot_slots=200,
                       positions=1, heads=16, seed=502, contexts=(3000, 1700))


def test_static_scratch_matches_the_allocating_step():
    log("no-alloc: larger workload, two positions")
    compare_workload(BIG)
    log("no-alloc: smaller workload after it (ragged, one position)")
    compare_workload(SMALL)


def test_static_scratch_in_every_copy_mode():
    import sparse_kv_offload_amd as sko
    for name, flags in (("late", sko.SKO_FLAG_LATE_COPY), ("fused", sko.SKO_FLAG_FUSED_COPY),
                        ("c8", sko.SKO_FLAG_INDEXER_C8), ("xcd_split", sko.SKO_FLAG_XCD_SPLIT)):
        log(f"no-alloc: {name}")
        compare_workload(SMALL.replace(name=f"noalloc_{name}"), flags)


def test_static_scratch_rejects_a_step_that_does_not_fit():
    """32 sequences x 8 positions x 45 000 tokens of candidates need more
    than the static area; the call fails before enqueueing anything."""
    import torch
    import sparse_kv_offload_amd as sko
    cfg = sko.make_config(num_layers=1, batch=32, max_tokens=45000, num_heads=1, top_k=16, hot_slots=128,
                          mtp_positions=8)
    with sko.SparseKVOffload(cfg, None) as h:
        qi = torch.zeros((32, 8, 64), dtype=torch.int16, device="cuda")
        qa = torch.zeros((32, 8, 1, 576), dtype=torch.int16, device="cuda")
        out = torch.zeros((32, 8, 1, 512), dtype=torch.float32, device="cuda")
        with pytest.raises(sko.SkoError) as e:
            sko.sko_decode_step_static(h.handle, 0, qi, qa, out)
        assert e.value.code == sko.SKO_E_UNSUPPORTED and "static" in str(e.value)
        assert h.stats(0).steps == 0  # nothing ran
