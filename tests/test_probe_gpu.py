"""GPU: the two bandwidth probes the benchmark reports its rates against
(kvd_hbm_read_probe for device memory, kvd_link_probe for the host link) run
and return rates inside what the hardware can do."""
import pytest

from decode_attention_offloaded_amd import kvd

pytestmark = pytest.mark.gpu


def test_hbm_read_probe_rate_is_plausible():
    g = kvd.hbm_read_probe(256 << 20, 3)
    print("device-memory read, 256 MiB: %.1f GB/s" % g)
    assert 500.0 < g < 10000.0  # MI355X: 8 TB/s peak


def test_link_probe_rate_is_plausible():
    g = kvd.link_probe(64 << 20, 2, 3)
    print("pinned host to device, 64 MiB over 2 streams: %.2f GB/s" % g)
    assert 1.0 < g < 200.0
