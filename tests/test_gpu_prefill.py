"""Layerwise prefill offload on the GPU through the C ABI, against the
oracle's pass replay: every layer's compute sees exactly its own KV so far in
its buffer (even though the buffers are shared), and the host pool ends with
every layer's prefix followed by each pass's new rows, byte for byte, for
several lookaheads and buffer counts."""
import numpy as np
import pytest

from oracle import prefill as P

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


class DeviceBytes:
    """A device address seen by torch as a uint8 tensor (no copy)."""

    def __init__(self, ptr: int, nbytes: int):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False),
                                         "version": 3, "strides": None, "stream": None}


def run_case(n, indep, shared, lookahead, passes, row_bytes=64, capacity=48, seed=0):
    import torch
    import sparse_kv_offload_amd as sko
    rng = np.random.default_rng(seed)
    stream = torch.cuda.current_stream()
    pre = [rng.integers(0, 256, size=(int(rng.integers(0, 8)), row_bytes), dtype=np.uint8) for _ in range(n)]
    new = [[rng.integers(0, 256, size=(int(rng.integers(1, 5)), row_bytes), dtype=np.uint8) for _ in range(n)]
           for _ in range(passes)]
    with sko.PrefillOffload(n, shared, lookahead, row_bytes, capacity, independent=indep, stream=stream) as pf:
        buf_of, nphys = pf.plan()
        want_plan = P.plan([0] * n, indep, shared, [capacity * row_bytes] * n)
        assert buf_of.tolist() == want_plan["buffer_of_layer"] and nphys == want_plan["physical"]
        for l in range(n):
            pf.host_pool(l)[: len(pre[l])] = pre[l]
            pf.set_tokens(l, len(pre[l]))
        seen = []
        for c in range(passes):
            seen_c = []
            for l in range(n):
                ptr = pf.begin_layer(l)
                P_l = pf.tokens(l)
                buf = torch.as_tensor(DeviceBytes(ptr, capacity * row_bytes), device="cuda")
                # the layer's compute: read its KV so far, write its new rows after it
                seen_c.append(buf[: P_l * row_bytes].clone())
                rows = torch.from_numpy(new[c][l].reshape(-1)).to("cuda", non_blocking=False)
                buf[P_l * row_bytes:(P_l + len(new[c][l])) * row_bytes].copy_(rows)
                pf.end_layer(l, len(new[c][l]))
            seen.append(seen_c)
        pf.sync()
        host_o, seen_o = P.run_passes(n, want_plan["buffer_of_layer"], want_plan["dedicated"], capacity,
                                      row_bytes, pre, new)
        for l in range(n):
            t = pf.tokens(l)
            assert t == len(host_o[l])
            assert np.array_equal(pf.host_pool(l)[:t], host_o[l]), f"host pool of layer {l}"
        for c in range(passes):
            for l in range(n):
                got = seen[c][l].cpu().numpy().reshape(-1, row_bytes)
                assert np.array_equal(got, seen_o[c][l]), f"pass {c} layer {l} saw other rows"
        timing = [pf.layer_timing(l) for l in range(n)]
    return timing


@pytest.mark.parametrize("lookahead", [1, 2, 3, 6])
def test_four_trays(lookahead):
    """The explainer's layout: B0 bound to layer 0, three rotating trays."""
    n = 9
    log(f"case prefill trays lookahead={lookahead}")
    run_case(n, [1] + [0] * (n - 1), 3, lookahead, passes=3, seed=lookahead)


@pytest.mark.parametrize("shared", [1, 2, 5])
def test_shared_buffer_counts(shared):
    n = 7
    log(f"case prefill shared={shared}")
    run_case(n, [1, 0, 0, 1, 0, 0, 0], shared, 2, passes=2, seed=10 + shared)


def test_out_of_order_is_rejected():
    import torch
    import sparse_kv_offload_amd as sko
    with sko.PrefillOffload(4, 2, 1, 64, 8, stream=torch.cuda.current_stream()) as pf:
        with pytest.raises(sko.SkoError) as e:
            pf.begin_layer(1)
        assert e.value.code == sko.SKO_E_STATE
        pf.begin_layer(0)
        with pytest.raises(sko.SkoError) as e:
            pf.end_layer(0, 9)
        assert e.value.code == sko.SKO_E_CAPACITY
        pf.end_layer(0, 1)
        with pytest.raises(sko.SkoError) as e:
            pf.set_tokens(2, 1)
        assert e.value.code == sko.SKO_E_STATE
        for l in range(1, 4):
            pf.begin_layer(l)
            pf.end_layer(l, 0)
        pf.sync()
        assert [pf.tokens(l) for l in range(4)] == [1, 0, 0, 0]
