"""GPU parity of the quantisation kernels: bit-exact codes and scales.

The HIP kernels (through the C ABI) and the CPU oracle quantise the same
seeded inputs; every code byte and every fp32 scale bit must match.
"""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
import workloads
from oracle import quant_act_ref, quant_weight_ref
from helpers import to_gpu

pytestmark = pytest.mark.gpu


def _act_gpu(a_bf16: torch.Tensor):
    a_q, a_s = fp8bq.quant_act(to_gpu(a_bf16))
    torch.cuda.synchronize()
    return a_q.cpu().numpy(), a_s.cpu().numpy()


def _assert_bitexact(got, want, what):
    gq, gs = got
    wq, ws = want
    assert gq.shape == wq.shape and gs.shape == ws.shape, what
    bad = np.nonzero(gq != wq)
    assert bad[0].size == 0, f"{what}: {bad[0].size} code mismatches, first at {[b[0] for b in bad]}: gpu {gq[tuple(b[0] for b in bad)]:#x} oracle {wq[tuple(b[0] for b in bad)]:#x}"
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32)), f"{what}: scale bits differ"


def test_quant_act_tiny_case():
    a, _ = workloads.tiny_inputs()
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), "tiny")


@pytest.mark.parametrize("k", [3072, 5120, 8704])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 7, 8, 16, 33, 64])
def test_quant_act_decode_verify_batch_shapes(m, k):
    a = workloads.activation(m, 5120, k)
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), f"M={m} K={k}")


@pytest.mark.parametrize("n,k", workloads.PREFILL_SHAPES)
def test_quant_act_prefill(n, k):
    a = workloads.activation(workloads.PREFILL_M, n, k)
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), f"prefill K={k}")


def test_quant_act_adversarial_groups():
    # golden-style ties, signed zeros, subnormal results, tiny and huge
    # magnitudes (bf16 has fp32's exponent range), one group per row
    rows = []
    g = np.zeros(128, np.float32)
    g[:8] = [448, 1.0625, 1.1875, 432, 2 ** -10, 3 * 2 ** -10, 2 ** -10 * (1 + 2 ** -7), -1.0625]
    rows.append(g)
    rows.append(np.array([1.53125, 1.3671875] + [0] * 126, np.float32))  # x/s exactly a tie
    rows.append(np.full(128, -0.0, np.float32))
    rows.append(np.zeros(128, np.float32))
    rows.append(np.full(128, 3.0, np.float32))
    rows.append((np.arange(128, dtype=np.float32) - 64) * np.float32(2.0 ** -120))  # tiny, fp32-normal
    rows.append((np.arange(128, dtype=np.float32) - 64) * np.float32(2.0 ** 100))
    rng = np.random.default_rng(5)
    r = rng.standard_normal(128).astype(np.float32)
    r[17] = 3e4
    rows.append(r)  # one outlier flushes most codes to subnormals
    a = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), "adversarial")


def test_quant_act_random_bf16_bit_patterns():
    # every finite bf16 bit pattern class: random 16-bit words, NaN/Inf removed
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 16, size=(64, 1024), dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits[exp == 0xFF] &= 0x807F  # turn Inf/NaN into subnormals/zero of either sign
    a = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), "random bit patterns")


def _band_groups():
    """Groups whose first entry is a chosen maximum a and whose other
    entries run over every bf16 value x with a * 2^-19 <= |x| <= a, both
    signs (everything that quantises to a non-zero code, and the first
    values that round to zero), for about a thousand maxima: every exponent
    field 0..254 with mantissa fields 0x00, 0x01, 0x40, 0x7f (subnormal
    maxima included, zero excluded). Returns bf16 [rows, 8192]."""
    pos = np.arange(1, 0x7F80, dtype=np.uint32)  # positive finite bf16 patterns
    vals = (pos << 16).view(np.float32)
    groups = []
    for e in range(0, 255):
        for mant in (0x00, 0x01, 0x40, 0x7F):
            p = (e << 7) | mant
            if p == 0:
                continue
            a = np.float32(((np.uint32(p) << 16)).view(np.float32))
            sel = pos[(vals <= a) & (vals >= a * np.float32(2.0 ** -19))]
            xs = np.concatenate([sel, sel | 0x8000]).astype(np.uint16)
            n_g = -(-xs.size // 127)
            body = np.zeros(n_g * 127, dtype=np.uint16)
            body[: xs.size] = xs
            g = np.empty((n_g, 128), dtype=np.uint16)
            g[:, 0] = p
            g[:, 1:] = body.reshape(n_g, 127)
            groups.append(g)
    g = np.concatenate(groups)
    rows = -(-g.shape[0] // 64)
    out = np.zeros((rows * 64, 128), dtype=np.uint16)
    out[: g.shape[0]] = g
    return torch.from_numpy(out.reshape(rows, 64 * 128).view(np.int16)).view(torch.bfloat16)


def test_quant_act_every_bf16_value_under_a_thousand_maxima():
    # the kernel forms x / s from the reciprocal of s and one fma correction
    # (IEEE division only below amax = 2^-96); its codes must still be those
    # of the correctly rounded division for every input it can see
    a = _band_groups()
    _assert_bitexact(_act_gpu(a), quant_act_ref(a), "bf16 values under chosen maxima")


def test_quant_act_empty_is_noop():
    a_q, a_s = fp8bq.quant_act(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert a_q.shape == (0, 256) and a_s.shape == (0, 2)


def _weight_gpu(w: np.ndarray):
    w_q, w_s = fp8bq.quant_weight(to_gpu(w))
    torch.cuda.synchronize()
    return w_q.cpu().numpy(), w_s.cpu().numpy()


def test_quant_weight_tiny_case():
    _, w = workloads.tiny_inputs()
    _assert_bitexact(_weight_gpu(w), quant_weight_ref(w), "tiny weight")


@pytest.mark.parametrize("n,k", [(200, 256), (17, 384), (129, 128), (1000, 640)])
def test_quant_weight_ragged_row_blocks(n, k):
    w = workloads.weight(n, k)
    w[n - 1, k - 1] = 0.75  # outlier in the short last block
    _assert_bitexact(_weight_gpu(w), quant_weight_ref(w), f"N={n} K={k}")


@pytest.mark.parametrize("n,k", workloads.SHAPES)
def test_quant_weight_full_shapes_sampled_blocks(n, k):
    # full-size W on the GPU; the oracle re-derives a few row blocks (first,
    # last, two inside) from the per-block seeds and must match bit for bit
    w = workloads.weight(n, k)
    gq, gs = _weight_gpu(w)
    nb = (n + 127) // 128
    for b in sorted({0, 1, nb // 2, nb - 1}):
        oq, os_ = quant_weight_ref(workloads.weight_block(n, k, b))
        assert np.array_equal(gq[128 * b : 128 * b + 128], oq), f"codes of block row {b}"
        assert np.array_equal(gs[b : b + 1].view(np.uint32), os_.view(np.uint32)), f"scales of block row {b}"
