"""Pins of the layerwise prefill offload oracle (oracle/prefill.py), CPU only.

Against what the pages fix: the closed form physical = I + min(B, R) of a
uniform layout and its footprint ratio; the explainer's four trays for a
78-layer model (B0 bound to layer 0, B1..B3 rotating, about 4/78 = 5.1 % of
the fully resident K/V); no sharing across incompatible specifications;
failing validation; the exposed-delay model; and data invariants of the
pass replay (every layer's compute sees exactly its own prior KV, the host
ends with the prefix followed by every pass's new rows).  The planted
mistakes at the end must each be rejected by some pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import prefill as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_trays_78.json")


def pin_closed_form_uniform():
    for n in range(1, 40):
        for i in range(0, n + 1):
            for b in range(1, 6):
                r = P.plan([7] * n, [1] * i + [0] * (n - i), b, [64] * n)
                assert r["physical"] == P.closed_form_uniform(n, i, b) == i + min(b, n - i)
                assert abs(r["footprint_ratio"] - r["physical"] / n) < 1e-12


def pin_four_trays_of_the_explainer():
    g = json.load(open(GOLDEN))
    n = g["layers"]
    r = P.plan([0] * n, [1] + [0] * (n - 1), g["rotating_trays"], [1152] * n)
    assert r["physical"] == g["trays"]
    assert round(100.0 * r["footprint_ratio"], 1) == g["footprint_percent"]
    b = r["buffer_of_layer"]
    assert b[0] == 0 and all(x != 0 for x in b[1:])          # B0 stays bound to layer 0
    assert [b[l] for l in range(1, 7)] == [1, 2, 3, 1, 2, 3]  # B1..B3 rotate


def pin_no_sharing_across_specs():
    specs = [0, 1, 0, 1, 1, 0, 2, 0]
    r = P.plan(specs, [0] * 8, 2, [10, 20, 10, 20, 20, 10, 30, 10])
    b = r["buffer_of_layer"]
    for l in range(8):
        for m in range(8):
            if specs[l] != specs[m]:
                assert b[l] != b[m]
    # each group: min(B, R_g) buffers, layers in round-robin order
    assert [b[l] for l in (0, 2, 5, 7)] == [0, 1, 0, 1]
    assert [b[l] for l in (1, 3, 4)] == [2, 3, 2]
    assert b[6] == 4 and r["physical"] == 5


def pin_validation():
    for args in (([0, 0], [0, 0], 0, [1, 1]), ([0], [2], 1, [1]), ([0], [0], 1, [0]),
                 ([0, 0], [0, 0], 1, [1, 2]), ([], [], 1, [])):
        with pytest.raises(P.PlanError):
            P.plan(*args)
    assert P.plan([0, 0], [1, 1], 0, [1, 1])["physical"] == 2  # no reusable layer needs no shared buffer


def pin_exposed_delay():
    assert P.exposed_delay(3.0, 1.0) == 2.0
    assert P.exposed_delay(1.0, 3.0) == 0.0
    assert P.exposed_delay(2.0, 2.0) == 0.0


def pin_pass_replay():
    rng = np.random.default_rng(3)
    for n, i, b in ((6, 1, 3), (9, 2, 2), (5, 0, 1)):
        r = P.plan([0] * n, [1] * i + [0] * (n - i), b, [1] * n)
        prefix = [rng.integers(0, 1 << 16, size=(int(rng.integers(1, 5)), 3), dtype=np.uint16) for _ in range(n)]
        passes = [[rng.integers(0, 1 << 16, size=(2, 3), dtype=np.uint16) for _ in range(n)] for _ in range(3)]
        host, seen = P.run_passes(n, r["buffer_of_layer"], r["dedicated"], 32, 3, prefix, passes)
        for l in range(n):
            want = np.concatenate([prefix[l]] + [passes[c][l] for c in range(3)])
            assert np.array_equal(host[l], want)
            for c in range(3):
                before = np.concatenate([prefix[l]] + [passes[d][l] for d in range(c)])
                assert np.array_equal(seen[c][l], before), (n, i, b, c, l)


PINS = [pin_closed_form_uniform, pin_four_trays_of_the_explainer, pin_no_sharing_across_specs, pin_validation,
        pin_exposed_delay, pin_pass_replay]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    P.set_mutation("")
    pin()


@pytest.mark.parametrize("mutation", P.MUTATIONS)
def test_planted_mistakes(mutation):
    P.set_mutation(mutation)
    try:
        caught = []
        for pin in PINS:
            try:
                pin()
            except (AssertionError, P.PlanError):
                caught.append(pin.__name__)
        assert caught, f"no pin rejects {mutation}"
    finally:
        P.set_mutation("")
