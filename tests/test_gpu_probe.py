"""The read-ceiling probe kernels through the C ABI: they read the whole
buffer (or every listed tile) and write nothing but the sink, which stays zero
unless a workgroup's xor of what it read equals the probes' never-value."""
import pytest
import torch

from paged_kv_cache_260_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


@pytest.mark.parametrize("grid", [1, 7, 256])
def test_stream_read_probe(grid):
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")     # 1 MiB, every 16-byte unit distinct
    before = buf.clone()
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    _lib.probe_stream_read(buf, grid, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("depth", [1, 2, 4])
def test_gather_tiles_probe(depth):
    pool = torch.arange(64 * 1024, dtype=torch.int32, device="cuda")   # 64 tiles of 4 KiB
    tiles = torch.randperm(64, device="cuda").to(torch.int32)
    tiles = torch.cat([tiles, torch.tensor([-5, 1000], dtype=torch.int32, device="cuda")])  # clamped, never out of bounds
    before = pool.clone()
    sink = torch.zeros(32, dtype=torch.int32, device="cuda")
    _lib.probe_gather_tiles(pool, tiles, depth, 32, sink)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    assert int(sink.abs().sum()) == 0
