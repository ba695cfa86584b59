"""The measurement kernels behind the roofline denominators read and compute
what they claim: the streaming read touches every 32-bit word exactly once
(its XOR words combine to the XOR of the whole buffer, computed on the CPU),
and the MFMA loop's sums equal the closed form 4096 * iters * dec(code)^2."""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 1 << 20, (1 << 20) + 48, 40_000_016])
@pytest.mark.parametrize("grid", [7, 256])
def test_read_touches_every_word_once(nbytes, grid):
    rng = np.random.default_rng([nbytes, grid])
    host = rng.integers(-(1 << 31), 1 << 31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = fp8bq.mb_read(buf, grid=grid)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy()) if grid > 0 else 0
    want = np.bitwise_xor.reduce(host) if host.size else np.int32(0)
    assert int(got) == int(want)
    if nbytes == 0:
        assert torch.all(sink == 0)


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0x30, 0.5), (0xB8, -1.0), (0x01, 2.0 ** -9)])
def test_mfma_loop_closed_form(code, value):
    iters = 100
    sink = fp8bq.mb_mfma(grid=3, iters=iters, code=code)
    torch.cuda.synchronize()
    assert torch.all(sink == 4096.0 * iters * value * value)


def test_empty_launch():
    for _ in range(10):
        fp8bq.mb_empty(256, 512)
    torch.cuda.synchronize()
