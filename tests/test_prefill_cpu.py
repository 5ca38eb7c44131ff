"""The prefill buffer planner of libsko (host code, no GPU needed) against
the oracle's planner, and argument validation of the prefill calls."""
import numpy as np
import pytest

from oracle import prefill as P


def test_library_plan_matches_oracle():
    import sparse_kv_offload_amd as sko
    rng = np.random.default_rng(31)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        nspec = int(rng.integers(1, 4))
        specs = rng.integers(0, nspec, n).tolist()
        size_of = {s: int(rng.integers(1, 1 << 20)) for s in range(nspec)}
        sizes = [size_of[s] for s in specs]
        indep = (rng.random(n) < 0.2).astype(int).tolist()
        b = int(rng.integers(1, 6))
        want = P.plan(specs, indep, b, sizes)
        got, nphys = sko.sko_prefill_plan(specs, indep, b, sizes)
        assert got.tolist() == want["buffer_of_layer"] and nphys == want["physical"]


def test_explainer_trays():
    import sparse_kv_offload_amd as sko
    buf, nphys = sko.sko_prefill_plan([0] * 78, [1] + [0] * 77, 3, [1152 * 4096] * 78)
    assert nphys == 4 and buf[0] == 0 and buf[1:7].tolist() == [1, 2, 3, 1, 2, 3]


@pytest.mark.parametrize("args", [
    ([0, 0], [0, 0], 0, [1, 1]),      # reusable layers, no shared buffer
    ([0], [2], 1, [1]),               # bad flag
    ([0], [0], 1, [0]),               # size 0
    ([0, 0], [0, 0], 1, [1, 2]),      # one spec, two sizes
    ([0], [0], -1, [1]),              # B < 0
])
def test_library_plan_rejects(args):
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_prefill_plan(*args)
    assert e.value.code == sko.SKO_E_INVAL
    with pytest.raises(P.PlanError):
        P.plan(*args)


@pytest.mark.parametrize("bad", [dict(num_layers=0), dict(shared_buffers=0), dict(lookahead=0),
                                 dict(row_bytes=24), dict(row_bytes=0), dict(capacity_tokens=0),
                                 dict(device=-1)])
def test_create_rejects_bad_config(bad):
    import sparse_kv_offload_amd as sko
    base = dict(num_layers=4, shared_buffers=3, lookahead=1, row_bytes=64, capacity_tokens=16, device=0)
    base.update(bad)
    with pytest.raises(sko.SkoError) as e:
        sko.PrefillOffload(**base)
    assert e.value.code == sko.SKO_E_INVAL
