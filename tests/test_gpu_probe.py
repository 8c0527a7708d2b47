"""The streaming-read probe (a measurement companion): runs on buffers of any 16-byte multiple,
including a ragged tail, and leaves its sink alone for a buffer whose XOR-fold is not the
sentinel."""
import pytest
import torch

from paged_kv_cache_416_amd import kernels

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_read_probe_runs(nbytes):
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    kernels.read_probe(src, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
