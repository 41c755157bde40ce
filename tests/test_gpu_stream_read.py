"""The streaming-read measurement kernel reads every byte of its buffer once: the word each
workgroup writes equals the xor of the 32-bit words of the 8 KB blocks it owns (block q belongs
to workgroup q % G), bit-exact, also for a buffer that ends inside a block."""
import numpy as np
import pytest
import torch

import mixture_experts_forward_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 1000, (64 << 20) // 16 + 3])
def test_stream_read_xor_of_shares(n16):
    g = torch.Generator(device="cpu").manual_seed(1234 + n16)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), generator=g, dtype=torch.int32)
    buf = host.to("cuda:0")
    sink = moe.moe_stream_read(buf)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = host.numpy().view(np.uint32).reshape(n16, 4)
    grid = got.size
    block = 512  # 16-byte units per block (one per thread of a workgroup)
    owner = (np.arange(n16) // block) % grid
    want = np.zeros(grid, np.uint32)
    per_unit = np.bitwise_xor.reduce(words, axis=1)
    for b in range(grid):
        sel = per_unit[owner == b]
        want[b] = np.bitwise_xor.reduce(sel) if sel.size else np.uint32(0)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "workgroups %s of %d" % (bad[:5], grid)
