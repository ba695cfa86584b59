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


# Operands from memory: small codes (0, +-0.5, +-1, +-2) keep every sum
# exact in fp32, so the GPU's per-thread sums must equal the closed form of
# the documented operand layout: lane l's element i (row r = 4 (l / 16) + i,
# column c = l % 16) sums dec(first[16 q + r][b]) * dec(second[16 q + c][b])
# over q = 0..3 and byte b = 0..31.
def test_mfma_data_loop_matches_its_operands():
    from oracle import e4m3_decode

    rng = np.random.default_rng(11)
    codes = rng.choice(np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8),
                       size=fp8bq.MB_MFMA_DATA_BYTES)
    iters, grid = 37, 5
    sink = fp8bq.mb_mfma_data(grid, iters, torch.from_numpy(codes).cuda())
    torch.cuda.synchronize()
    dec = e4m3_decode(codes).reshape(8, 2, 64, 32)  # chain, operand, lane, byte
    want = np.zeros(64)
    for lane in range(64):
        for i in range(4):
            r, c = 4 * (lane // 16) + i, lane % 16
            for u in range(8):
                want[lane] += sum(float(np.dot(dec[u, 0, 16 * q + r], dec[u, 1, 16 * q + c])) for q in range(4))
    got = sink.cpu().numpy().reshape(grid * 4, 64)
    assert np.array_equal(got, np.broadcast_to((iters * want).astype(np.float32), got.shape))


def test_mfma_scaled_loop_is_scale_times_the_plain_loop():
    # the block-scaled inner loop (fresh products, 4 scale FMAs each, one
    # MFMA later) against the closed form: scale times the plain loop's sums;
    # codes in {0, +-0.5, +-1, +-2} and scale 0.75 keep every value exact
    from oracle import e4m3_decode

    rng = np.random.default_rng(12)
    codes = rng.choice(np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8),
                       size=fp8bq.MB_MFMA_DATA_BYTES)
    iters, grid, scale = 29, 3, 0.75
    sink = fp8bq.mb_mfma_scaled(grid, iters, torch.from_numpy(codes).cuda(), scale)
    torch.cuda.synchronize()
    dec = e4m3_decode(codes).reshape(8, 2, 64, 32)  # chain, operand, lane, byte
    want = np.zeros(64)
    for lane in range(64):
        for i in range(4):
            r, c = 4 * (lane // 16) + i, lane % 16
            for u in range(8):
                want[lane] += sum(float(np.dot(dec[u, 0, 16 * q + r], dec[u, 1, 16 * q + c])) for q in range(4))
    got = sink.cpu().numpy().reshape(grid * 4, 64)
    assert np.array_equal(got, np.broadcast_to((scale * iters * want).astype(np.float32), got.shape))
    # zero iterations: nothing accumulated
    sink = fp8bq.mb_mfma_scaled(grid, 0, torch.from_numpy(codes).cuda(), scale)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)


def test_empty_launch():
    for _ in range(10):
        fp8bq.mb_empty(256, 512)
    torch.cuda.synchronize()
