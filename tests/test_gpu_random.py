"""Randomized parity sweep: seeded random configurations (batch up to 8,
ragged contexts from one token to 20 000, k above and below the context up
to 1000, one to four positions, head counts that leave partial head groups,
shelf sizes at and above D*k, query drift with and without topic jumps, one
or two layers)
under every valid combination of the copy arrangement, the int8 indexer and
the split attention.  Each case runs all its (layer, sequence) chains
against the oracle to the full bar (selection, tables, hot-buffer bytes,
attention)."""
import numpy as np
import pytest

import synth
from parity_harness import run_parity

pytestmark = pytest.mark.gpu

N_CASES = 64


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_kv_offload_amd  # noqa: F401
    yield


def random_case(i):
    import sparse_kv_offload_amd as sko
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 9))
    D = int(rng.integers(1, 5))
    H = int(rng.choice([1, 3, 16, 17, 20, 32]))
    k = int(rng.choice([16, 40, 64, 100, 256, 512, 1000]))
    contexts = tuple(int(rng.choice([1, 7, int(rng.integers(8, 300)), int(rng.integers(300, 5000)),
                                     int(rng.integers(5000, 20000))]))
                     for _ in range(B))
    S = D * k + int(rng.integers(0, 3)) * int(rng.integers(1, 200))
    drift = [(0.9, 0.1), (0.5, 0.5), (0.95, 0.05)][int(rng.integers(0, 3))]
    w = synth.Workload(f"rand{i}", layers=int(rng.integers(1, 3)), batch=B, context=max(contexts),
                       contexts=contexts, steps=int(rng.integers(3, 6)), top_k=k, hot_slots=S, positions=D,
                       heads=H, drift=drift, jump_every=int(rng.choice([0, 2])), seed=int(rng.integers(1, 1 << 30)))
    modes = ["early", "late"] + (["fused"] if D == 1 and H <= 16 else [])
    mode = modes[int(rng.integers(0, len(modes)))]
    flags = {"early": 0, "late": sko.SKO_FLAG_LATE_COPY, "fused": sko.SKO_FLAG_FUSED_COPY}[mode]
    if rng.random() < 0.4:
        flags |= sko.SKO_FLAG_INDEXER_C8
    if mode == "early" and rng.random() < 0.4:
        flags |= sko.SKO_FLAG_HIT_OVERLAP
    return w, flags, mode


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config(i):
    w, flags, mode = random_case(i)
    log(f"random case {i}: L={w.layers} B={w.batch} contexts={w.contexts} D={w.positions} H={w.heads} "
        f"k={w.top_k} S={w.hot_slots} steps={w.steps} drift={w.drift} jump={w.jump_every} copy={mode} "
        f"flags={flags:#x}")
    worst = run_parity(w, check_keys=False, flags=flags, log=None)
    log(f"random case {i}: ok, attention worst {worst}")
