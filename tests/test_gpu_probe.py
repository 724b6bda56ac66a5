"""The read-bandwidth probe (moe_read_probe) reads every byte of its buffer:
the XOR of its sink words equals the XOR of the buffer's 32-bit words."""
import numpy as np
import pytest
import torch

import sparse_moe_feed_amd as moe
from gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_read_probe_checksum(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    announce(f"read probe {nbytes} bytes")
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = moe.read_probe(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
