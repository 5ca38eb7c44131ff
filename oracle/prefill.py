"""CPU oracle for layerwise prefill offload: buffer planning and the data
each layer's tray and the host pool hold.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers; the product path never
imports this module.

Follows "Layerwise and Sparse KV Cache Offloading Design" (vLLM-Ascend
design doc), section 3 "Layerwise Prefill Offload": buffer planning (the
closed form for a uniform layout, round-robin sharing, no sharing across
incompatible specifications, validation before use), the per-layer
execution pipeline (load the cached prefix, wait until the buffer is safe,
compute and update, save, prefetch a later layer) and the reuse invariant;
and the FlashOffloading explainer's prefill paragraphs (four trays: B0
bound to layer 0, B1..B3 rotating; onload_layer_map sets how far ahead
layers load; exposed delay per layer = max(0, transfer - compute)).

Readings where the pages leave a point open:
  * independent layers get dedicated buffers, numbered first in layer order;
  * reusable layers are grouped by specification (first appearance order);
    group g of R_g layers owns min(B, R_g) shared buffers, and its r-th
    layer (layer order) takes buffer r mod min(B, R_g) of the group; so a
    uniform layout gives I + min(B, R) buffers;
  * B = 0 with reusable layers, a non-positive size, or an independent
    flag other than 0/1 is an invalid plan (rejected, nothing planned);
  * a pass over the layers loads each layer's cached prefix into its
    buffer unless the buffer is dedicated and already holds it, lets the
    layer compute write its new rows after the prefix, and saves exactly
    those new rows to the host at the prefix end.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np


class PlanError(ValueError):
    pass


# Planted-mistake switch (empty in every real use; the pin tests set it to
# show that each pin rejects a plausible slip here).
_MUTATION = ""


def set_mutation(name: str = "") -> None:
    global _MUTATION
    _MUTATION = name or ""


MUTATIONS = ("one_shared_buffer", "share_across_specs", "never_reload", "reload_dedicated_skipped_always",
             "min_dropped")


def plan(specs: Sequence[int], independent: Sequence[int], shared: int, sizes: Sequence[int]) -> Dict:
    """Buffer of every layer.  specs[l]: specification id of layer l
    (equal ids = compatible layouts); independent[l] in {0, 1}; shared: B;
    sizes[l]: bytes of layer l's buffer (equal within a spec)."""
    n = len(specs)
    if n < 1 or len(independent) != n or len(sizes) != n or shared < 0:
        raise PlanError("bad shape")
    for l in range(n):
        if independent[l] not in (0, 1) or sizes[l] <= 0:
            raise PlanError(f"layer {l}: bad flag or size")
    for l in range(n):
        for m in range(l):
            if specs[l] == specs[m] and sizes[l] != sizes[m]:
                raise PlanError(f"layers {m} and {l}: one spec, two sizes")
    buf = [-1] * n
    nxt = 0
    for l in range(n):
        if independent[l]:
            buf[l] = nxt
            nxt += 1
    groups: List[int] = []
    for l in range(n):
        if not independent[l] and specs[l] not in groups:
            groups.append(specs[l])
    if _MUTATION == "share_across_specs":
        groups = groups[:1]
    for g in groups:
        if _MUTATION == "share_across_specs":
            members = [l for l in range(n) if not independent[l]]
        else:
            members = [l for l in range(n) if not independent[l] and specs[l] == g]
        if shared == 0:
            raise PlanError("reusable layers but no shared buffer")
        nb = min(shared, len(members))
        if _MUTATION == "one_shared_buffer":
            nb = 1
        if _MUTATION == "min_dropped":
            nb = shared
        for r, l in enumerate(members):
            buf[l] = nxt + r % nb
        nxt += nb
    physical = nxt
    buffer_bytes = [0] * physical
    for l in range(n):
        buffer_bytes[buf[l]] = sizes[l]
    return {"buffer_of_layer": buf, "physical": physical,
            "footprint_ratio": sum(buffer_bytes) / float(sum(sizes)),
            "dedicated": [bool(independent[l]) for l in range(n)]}


def closed_form_uniform(n: int, i: int, b: int) -> int:
    """physical = I + min(B, R), R = N - I (uniform layout)."""
    return i + min(b, n - i)


def exposed_delay(transfer: float, compute: float) -> float:
    """Exposed delay of one layer: the transfer time not covered by the
    compute time available while it moves, never below zero."""
    return max(0.0, transfer - compute)


def run_passes(n_layers: int, buffer_of_layer: Sequence[int], dedicated: Sequence[bool], capacity: int,
               row_elems: int, prefix: Sequence[np.ndarray], new_rows: Sequence[Sequence[np.ndarray]]):
    """Replay passes (chunks) over the layers on explicit arrays.

    prefix[l]: [P_l][row_elems] rows already in the host pool of layer l;
    new_rows[c][l]: [C][row_elems] rows the layer's compute writes in pass c.
    Returns (host pools after all passes, the rows each layer's compute saw
    in its buffer before writing, per pass: [c][l] -> [P][row_elems])."""
    host = [np.array(prefix[l], copy=True) for l in range(n_layers)]
    nbuf = max(buffer_of_layer) + 1
    buffers = [np.zeros((capacity, row_elems), dtype=host[0].dtype) for _ in range(nbuf)]
    holder = [-1] * nbuf  # layer whose current KV a buffer holds
    seen = []
    for c, rows in enumerate(new_rows):
        seen_c = []
        for l in range(n_layers):
            b = buffer_of_layer[l]
            P = host[l].shape[0]
            reload = not (dedicated[l] and holder[b] == l)
            if _MUTATION == "never_reload":
                reload = holder[b] == -1
            if _MUTATION == "reload_dedicated_skipped_always":
                reload = not dedicated[l]
            if reload:
                buffers[b][:P] = host[l]          # load the cached prefix
            seen_c.append(buffers[b][:P].copy())
            C = rows[l].shape[0]
            if P + C > capacity:
                raise PlanError("buffer capacity exceeded")
            buffers[b][P:P + C] = rows[l]         # compute updates the KV
            host[l] = np.concatenate([host[l], rows[l]])  # save the new rows
            holder[b] = l
        seen.append(seen_c)
    return host, seen
