"""GPU checks of fp8bq_gemm_fused (activation quantisation inside the GEMM):
bitwise equal to fp8bq_quant_act followed by fp8bq_gemm, whose parity with
the oracle the other GPU tests establish, on ordinary, adversarial and
random-bit-pattern activations; plus one direct oracle comparison."""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
from helpers import assert_gemm_close, bf16_to_f64, to_gpu
from oracle import gemm_ref, quant_act_ref, quant_weight_ref
import workloads

pytestmark = pytest.mark.gpu


def _two_call(a_gpu, w_q, w_s):
    a_q, a_s = fp8bq.quant_act(a_gpu)
    return fp8bq.gemm(a_q, a_s, w_q, w_s)


def _check_bitwise(a: torch.Tensor, w_q, w_s, what):
    a_gpu = to_gpu(a)
    w_q, w_s = to_gpu(w_q), to_gpu(w_s)
    ref = _two_call(a_gpu, w_q, w_s)
    got = fp8bq.gemm_fused(a_gpu, w_q, w_s)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), what


def _weights(n, k):
    return quant_weight_ref(workloads.weight(n, k))


# every quantisation layout: 1, 2, 3..4 and 5..8 tokens
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(640, 1024), (700, 384), (130, 1152), (4100, 2304), (1000, 9216)])
def test_fused_bitwise_equals_two_calls(m, n, k):
    w_q, w_s = _weights(n, k)
    _check_bitwise(workloads.activation(m, n, k), w_q, w_s, f"M={m} N={n} K={k}")


def _adversarial(m, k, seed):
    """Groups built to stress the in-kernel quantiser: exact ties of the e4m3
    rounding after division, zeros and negative zeros, bf16 subnormals,
    groups with amax below 2^-96 (IEEE-division fallback), huge values,
    constant groups and one-hot groups."""
    rng = np.random.default_rng(seed)
    g = k // 128
    x = rng.standard_normal((m, k)).astype(np.float32)
    kinds = rng.integers(0, 8, size=(m, g))
    for i in range(m):
        for j in range(g):
            sl = slice(128 * j, 128 * j + 128)
            kind = kinds[i, j]
            if kind == 0:  # amax 448: quotient = x, codes at e4m3 ties (e.g. 1.0625 between 1 and 1.125)
                v = rng.choice(np.array([1.0625, -1.0625, 2.125, 3.25, -0.5625, 448.0], np.float32), 128)
                v[0] = 448.0
                x[i, sl] = v
            elif kind == 1:  # zeros with signs
                x[i, sl] = rng.choice(np.array([0.0, -0.0], np.float32), 128)
            elif kind == 2:  # tiny: below 2^-96, fallback path
                x[i, sl] *= np.float32(2.0 ** -110)
            elif kind == 3:  # bf16 subnormals
                x[i, sl] *= np.float32(2.0 ** -130)
            elif kind == 4:  # huge
                x[i, sl] *= np.float32(1e37)
            elif kind == 5:  # constant
                x[i, sl] = np.float32(rng.standard_normal())
            elif kind == 6:  # one-hot
                x[i, sl] = 0.0
                x[i, 128 * j + rng.integers(0, 128)] = np.float32(rng.standard_normal() * 5)
            # kind 7: plain Gaussian
    return torch.from_numpy(x).to(torch.bfloat16)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_fused_bitwise_adversarial(m):
    n, k = 520, 2048
    w_q, w_s = _weights(n, k)
    _check_bitwise(_adversarial(m, k, 100 + m), w_q, w_s, f"adversarial M={m}")


@pytest.mark.parametrize("m", [1, 2, 4, 8])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fused_bitwise_random_bf16_bit_patterns(seed, m):
    n, k = 300, 3072
    rng = np.random.default_rng([seed, m])
    bits = rng.integers(0, 1 << 16, size=(m, k), dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = np.where(finite, bits, bits & 0x807F)  # replace inf/nan by finite patterns
    a = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    w_q, w_s = _weights(n, k)
    _check_bitwise(a, w_q, w_s, f"random bit patterns seed={seed}")


def test_fused_against_oracle():
    m, n, k = 6, 700, 1536
    a = workloads.activation(m, n, k)
    w_q, w_s = _weights(n, k)
    c = bf16_to_f64(fp8bq.gemm_fused(to_gpu(a), to_gpu(w_q), to_gpu(w_s)))
    a_q, a_s = quant_act_ref(a)
    assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what="fused vs oracle")


@pytest.mark.parametrize("n,k", workloads.SHAPES)
def test_fused_full_size_bitwise(n, k):
    w_q, w_s = fp8bq.quant_weight(to_gpu(workloads.weight(n, k)))
    for m in (1, 2, 3, 4, 5, 8):
        a_gpu = to_gpu(workloads.activation(m, n, k))
        ref = _two_call(a_gpu, w_q, w_s)
        got = fp8bq.gemm_fused(a_gpu, w_q, w_s)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"M={m} N={n} K={k}"


def test_fused_rejects_more_than_8_tokens():
    w_q, w_s = _weights(256, 256)
    for m in (9, 16, 17):
        with pytest.raises(fp8bq.Fp8bqError):
            fp8bq.gemm_fused(to_gpu(workloads.activation(m, 256, 256)), to_gpu(w_q), to_gpu(w_s))
