"""The seeded input generator: known answers, distribution, determinism."""
import numpy as np

import synth


def test_splitmix64_known_answers():
    # published SplitMix64 outputs (state 0 and the common test seed 1234567)
    assert [int(x) for x in synth.splitmix64_sequence(0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert int(synth.splitmix64_sequence(1234567, 1)[0]) == 6457827717110365317


def test_normal_moments_and_bf16_rounding():
    key = synth.stream_key(1234, 9, 0, 0)
    z = synth.normal_f64(key, 0, 4096, 64).ravel()
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01
    # bf16 output is round-to-nearest-even of float32(z)
    b = synth.normal_bf16(key, 0, 4096, 64).ravel()
    f32 = z.astype(np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(b, want)
    # widening back is within half a bf16 ulp
    assert np.all(np.abs(synth.bf16_to_f32(b) - f32) <= np.abs(f32) * 2.0 ** -8 + 1e-38)


def test_rows_regenerate_independently():
    w = synth.TINY
    a = w.kv_rows(0, 0, 100, 50)
    b = w.kv_rows(0, 0, 0, 200)[100:150]
    assert np.array_equal(a, b)
    assert not np.array_equal(w.kv_rows(0, 0, 0, 4), w.kv_rows(0, 1, 0, 4))


def test_query_chain_recipe():
    w = synth.SMALL
    q = w.index_query_chain(0, 0)
    assert q.shape == (w.steps, 1, 64)
    n = np.linalg.norm(q[:, 0], axis=1)
    assert np.allclose(n, 1.0)
    cos = np.sum(q[1:, 0] * q[:-1, 0], axis=1)
    assert 0.6 < cos.mean() < 0.85  # drift 0.9 / 0.1 in 64 dims
    sh = synth.SHELF8.index_query_chain(0, 0)[:, 0]
    c = np.sum(sh[1:] * sh[:-1], axis=1)
    assert 0.85 < np.delete(c, [63, 127, 191]).mean() < 0.97
    assert np.all(np.abs(c[[63, 127, 191]]) < 0.6)  # topic jumps
    m = synth.MTP3.index_query_chain(0, 0, steps=8)
    assert m.shape == (8, 4, 64)
    cm = np.sum(m[:, 0] * m[:, 1], axis=1) / np.linalg.norm(m[:, 0], axis=1) / np.linalg.norm(m[:, 1], axis=1)
    assert 0.8 < cm.mean() < 0.98
