"""GPU parity of the weight-only block-FP8 GEMM (fp8bq_gemm_w8a16) against
the oracle's gemm_w8a16_ref, through the C ABI (bf16 activation, block-FP8
weights quantised by the oracle, or by the GPU at full size with the sampled
blocks checked bit-exact)."""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
from helpers import assert_gemm_close, bf16_to_f64, bf16_rne, to_gpu
from oracle import gemm_w8a16_ref, gemm_w8a16_ref_at, quant_weight_ref
import workloads

pytestmark = pytest.mark.gpu


def _run(a_bf16: torch.Tensor, w_q, w_s):
    c = fp8bq.gemm_w8a16(to_gpu(a_bf16), to_gpu(w_q), to_gpu(w_s))
    torch.cuda.synchronize()
    return bf16_to_f64(c)


def _problem(m, n, k):
    a = workloads.activation(m, n, k)  # bf16, seeded, with outliers
    w_q, w_s = quant_weight_ref(workloads.weight(n, k))
    return a, w_q, w_s


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 15, 16])
@pytest.mark.parametrize("n,k", [(640, 1024), (700, 384), (130, 1152), (4100, 2304), (1000, 9216), (17, 256)])
def test_w8a16_whole_output(m, n, k):
    a, w_q, w_s = _problem(m, n, k)
    c = _run(a, w_q, w_s)
    assert_gemm_close(c, gemm_w8a16_ref(a.float().numpy(), w_q, w_s), what=f"W8A16 M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 4, 8, 16])
def test_w8a16_integer_exact_bitwise(m):
    # integer activations |a| <= 8 (exact in bf16), codes |w| <= 8, weight
    # scales in {1/2, 1, 2}, K = 1024: every product, group sum and scaled
    # sum is a multiple of 1/2 below 2^17, exact in fp32 in any order, so
    # the bf16 output must equal the oracle's value rounded to bf16 exactly.
    n, k = 300, 1024
    rng = np.random.default_rng(m)
    a = torch.from_numpy(rng.integers(-8, 9, size=(m, k)).astype(np.float32)).to(torch.bfloat16)
    vals = np.arange(-8, 9, dtype=np.float32)
    from oracle import e4m3_encode_rne
    w_q = e4m3_encode_rne(rng.choice(vals, size=(n, k)))
    w_s = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=((n + 127) // 128, k // 128))
    c = _run(a, w_q, w_s)
    ref = gemm_w8a16_ref(a.float().numpy(), w_q, w_s)
    assert np.array_equal(c, bf16_rne(ref))


def test_w8a16_deterministic_and_k_zero():
    a, w_q, w_s = _problem(7, 2000, 2048)
    c1 = _run(a, w_q, w_s)
    c2 = _run(a, w_q, w_s)
    assert np.array_equal(c1, c2)
    z = fp8bq.gemm_w8a16(to_gpu(torch.zeros(3, 0, dtype=torch.bfloat16)), to_gpu(np.zeros((5, 0), np.uint8)),
                         to_gpu(np.zeros((1, 0), np.float32)))
    torch.cuda.synchronize()
    assert z.shape == (3, 5) and bool(torch.all(z == 0))


def test_w8a16_rejects_more_than_16_tokens():
    a, w_q, w_s = _problem(17, 256, 256)
    with pytest.raises(fp8bq.Fp8bqError):
        fp8bq.gemm_w8a16(to_gpu(a), to_gpu(w_q), to_gpu(w_s))


@pytest.fixture(scope="module")
def weights_on_gpu():
    cache = {}

    def get(n, k):
        if (n, k) not in cache:
            cache.clear()
            cache[(n, k)] = fp8bq.quant_weight(to_gpu(workloads.weight(n, k)))
        return cache[(n, k)]

    return get


@pytest.mark.parametrize("n,k", workloads.SHAPES)
@pytest.mark.parametrize("m", [1, 8, 16])
def test_w8a16_full_size_sampled(m, n, k, weights_on_gpu):
    w_q, w_s = weights_on_gpu(n, k)
    a = workloads.activation(m, n, k)
    c = bf16_to_f64(fp8bq.gemm_w8a16(to_gpu(a), w_q, w_s))
    rng = np.random.default_rng([m, n, k, 16])
    nb = (n + 127) // 128
    blocks = sorted({0, nb - 1, int(rng.integers(0, nb))})
    w_q_h = w_q.cpu().numpy()
    w_s_h = w_s.cpu().numpy()
    for b in blocks:
        # the GPU-quantised weight block equals the oracle's quantisation
        ow_q, ow_s = quant_weight_ref(workloads.weight_block(n, k, b))
        rows = slice(128 * b, min(128 * b + 128, n))
        assert np.array_equal(w_q_h[rows], ow_q) and np.array_equal(w_s_h[b], ow_s[0])
    cols = np.concatenate([np.arange(128 * b, min(128 * b + 128, n)) for b in blocks])
    rows = np.repeat(np.arange(m), len(cols))
    cols = np.tile(cols, m)
    ref = gemm_w8a16_ref_at(a.float().numpy(), w_q_h, w_s_h, rows, cols)
    full_rms = None  # bound taken on the sampled outputs' rms
    assert_gemm_close(c[rows, cols], ref, rms=full_rms, what=f"W8A16 M={m} N={n} K={k} (sampled)")
