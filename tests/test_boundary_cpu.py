"""The C-ABI library on a machine without a GPU: it loads, exports every
declared symbol, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for header in ("sko.h", "sko_prefill.h"):
        src = open(os.path.join(ROOT, "include", header)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(sko_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sko_create", "sko_append_token", "sko_decode_step", "sko_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import sparse_kv_offload_amd as sko
    lib = ctypes.CDLL(sko.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libsko.so does not export {name}"
    assert set(declared_functions()) == set(sko.EXPORTED)


def test_binding_names_match_the_abi():
    import sparse_kv_offload_amd as sko
    for name in declared_functions():
        assert callable(getattr(sko, name)), name


def good_cfg(sko, **kw):
    base = dict(num_layers=1, batch=2, max_tokens=1000, num_heads=16, top_k=64, hot_slots=256,
                mtp_positions=2)
    base.update(kw)
    return sko.make_config(**base)


@pytest.mark.parametrize("bad", [
    dict(index_dim=32), dict(kv_dim=512), dict(v_dim=576), dict(num_layers=0), dict(batch=0),
    dict(num_heads=0), dict(top_k=0), dict(mtp_positions=0), dict(max_tokens=0),
    dict(max_tokens=2 ** 31), dict(hot_slots=127), dict(attn_scale=0.0),
    dict(attn_scale=float("inf")), dict(attn_scale=float("nan")), dict(flags=0x800), dict(flags=0x60), dict(flags=0x110), dict(flags=0x120),
    dict(flags=0x30), dict(flags=0x50), dict(flags=0x80000000), dict(flags=3),
    dict(flags=0x10, mtp_positions=2), dict(flags=0x10, mtp_positions=1, num_heads=17),
    # the XCD split needs the early copy without the hit/miss split
    dict(flags=0x420), dict(flags=0x410), dict(flags=0x500),
    dict(device=-1),
])
def test_create_rejects_bad_config(bad):
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_create(good_cfg(sko, **bad))
    assert e.value.code == sko.SKO_E_INVAL
    assert sko.sko_last_error()


def test_create_rejects_unsupported_merge_width():
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_create(good_cfg(sko, top_k=4096, mtp_positions=3, hot_slots=3 * 4096))
    assert e.value.code == sko.SKO_E_UNSUPPORTED


def test_create_rejects_hot_rows_beyond_int32():
    """Hot rows of every layer (slot rows plus spare rows) are addressed by
    int32 row numbers: 2^14 layers x 2^9 sequences x 2^8 slots is refused."""
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_create(good_cfg(sko, num_layers=1 << 14, batch=1 << 9, hot_slots=1 << 8))
    assert e.value.code == sko.SKO_E_UNSUPPORTED


def test_calls_on_null_handle_fail_cleanly():
    import sparse_kv_offload_amd as sko
    import numpy as np
    lib = sko._lib
    assert lib.sko_append_token(None, 0, 0, None, None, 0, 0) == sko.SKO_E_INVAL
    assert lib.sko_decode_step(None, 0, None, None, None) == sko.SKO_E_INVAL
    assert lib.sko_decode_step_static(None, 0, None, None, None) == sko.SKO_E_INVAL
    assert lib.sko_decode_step_append(None, 0, None, None, None, None, None) == sko.SKO_E_INVAL
    buf = np.zeros(4, dtype=np.int32)
    assert lib.sko_read_step(None, 1, buf.ctypes.data, buf.nbytes) == sko.SKO_E_INVAL
    assert lib.sko_read_table(None, 0, 0, 1, buf.ctypes.data, buf.nbytes) == sko.SKO_E_INVAL
    assert lib.sko_set_timing(None, 1) == sko.SKO_E_INVAL
    n32, khz = ctypes.c_int32(), ctypes.c_double()
    assert lib.sko_get_copy_spans(None, None, 0, ctypes.byref(n32), ctypes.byref(khz)) == sko.SKO_E_INVAL
    d = ctypes.c_double()
    n = ctypes.c_int64()
    assert lib.sko_get_copy_overlap(None, ctypes.byref(d), ctypes.byref(d), ctypes.byref(d),
                                    ctypes.byref(n)) == sko.SKO_E_INVAL
    assert lib.sko_create(None, None, None) == sko.SKO_E_INVAL
    sko.sko_destroy(0)  # NULL is a no-op


def test_stage_names():
    import sparse_kv_offload_amd as sko
    names = [sko.sko_stage_name(i) for i in range(sko.sko_num_stages())]
    assert names[:3] == ["append_rows", "score_hist", "topk_filter"]
    assert "gather_misses" in names and "attn_partial" in names
    assert sko.sko_stage_name(99) == ""
    assert "gfx950" in sko.sko_version()


@pytest.mark.parametrize("args", [(-1, 1 << 20, 1), (0, 1 << 19, 1), (0, (1 << 20) + 8, 1), (0, 1 << 20, 0)])
def test_link_read_rate_rejects_bad_arguments(args):
    """Argument checks come before any device work (so they run without a GPU)."""
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_link_read_rate(*args)
    assert e.value.code == sko.SKO_E_INVAL


@pytest.mark.parametrize("args", [(-1, 32, 8192, 2048, 1), (0, 0, 8192, 2048, 1), (0, 32, 8192, 100, 1),
                                  (0, 32, 1000, 2048, 1), (0, 32, 8192, 2048, 0), (0, 1024, 8192, 2048, 1)])
def test_hbm_gather_rate_rejects_bad_arguments(args):
    """Argument checks come before any device work (so they run without a GPU)."""
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_hbm_gather_rate(*args)
    assert e.value.code == sko.SKO_E_INVAL


@pytest.mark.parametrize("args", [(-1, 1 << 28, 1), (0, 1000, 1), (0, (1 << 20) + 8, 1), (0, 1 << 28, 0),
                                  (0, (1 << 31) + 16, 1), (0, 1 << 28, 65)])
def test_hbm_read_rate_rejects_bad_arguments(args):
    """Argument checks come before any device work (so they run without a GPU)."""
    import sparse_kv_offload_amd as sko
    with pytest.raises(sko.SkoError) as e:
        sko.sko_hbm_read_rate(*args)
    assert e.value.code == sko.SKO_E_INVAL
