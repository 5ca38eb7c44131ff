"""The bandwidth probes on the GPU: a plausible host-link read rate for a
PCIe 5.0 x16 link (above 1 GB/s, below the link's 64 GB/s per direction plus
a margin), a plausible HBM rate for random whole-row gathers (above 0.5 TB/s,
below the 8 TB/s HBM3E peak plus a margin), and for a streaming read (above
2 TB/s, at most the peak plus a margin)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_link_read_rate_is_plausible():
    import sparse_kv_offload_amd as sko
    rate = sko.sko_link_read_rate(0, 256 << 20, 1)
    print(f"zero-copy read {rate:.1f} GB/s", flush=True)
    assert 1.0 < rate < 80.0


def test_hbm_gather_rate_is_plausible():
    import sparse_kv_offload_amd as sko
    rate = sko.sko_hbm_gather_rate(0, 8, 4096, 1024, 1)
    print(f"row gather {rate:.0f} GB/s", flush=True)
    assert 500.0 < rate < 9000.0


def test_hbm_read_rate_is_plausible():
    """A cold streaming read of 256 MiB lands between a fraction of the 8 TB/s
    HBM peak and the peak itself (each launch reads a buffer the previous
    three launches did not touch, 1 GiB in all, four times the on-die
    Infinity Cache)."""
    import sparse_kv_offload_amd as sko
    rate = sko.sko_hbm_read_rate(0, 1 << 28, 2)
    print(f"stream read {rate:.0f} GB/s", flush=True)
    assert 2000.0 < rate < 8500.0
