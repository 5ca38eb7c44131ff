"""The host-link read probe on the GPU: a plausible rate for a PCIe 5.0 x16
link (above 1 GB/s, below the link's 64 GB/s per direction plus a margin),
and the bulk-copy comparison the benchmark reports beside it."""
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
