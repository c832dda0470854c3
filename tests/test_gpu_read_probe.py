"""The read probe (a measurement aid beside the attention kernels): it streams a buffer, leaves
the caller's memory alone unless the XOR of the data happens to match its guard constant, and
reports its launch status."""

import pytest
import torch

from tests.gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 16 * 257, 64 << 20])
def test_read_probe_streams_without_writing(nbytes):
    K = require_gpu()
    announce(f"read probe {nbytes} bytes")
    buf = torch.full((nbytes,), 3, dtype=torch.uint8, device="cuda")   # every word 0x03030303
    sink = torch.full((4,), -5, dtype=torch.int32, device="cuda")
    K.kv_attn_read_probe(buf, sink)
    torch.cuda.synchronize()
    # an even number of equal words XORs to 0 per lane, never the guard constant: no store
    assert bool((sink == -5).all())
    assert bool((buf == 3).all())


def test_read_probe_binding_checks():
    K = require_gpu()
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        K.kv_attn_read_probe(buf, torch.zeros(1, dtype=torch.int16, device="cuda"))
    with pytest.raises(K.KvAttnError):
        K.kv_attn_read_probe(buf[:1000], torch.zeros(1, dtype=torch.int32, device="cuda"))
