"""GPU parity of the block-FP8 GEMM against the fp64 oracle.

Acceptance: |C_gpu - C_ref| <= 1e-2 * rms(C_ref) + 2^-8 * |C_ref| for every
output (fp32 accumulation in any order plus one bf16 rounding); bit-exact
bf16 where all partial sums are exact in fp32 (integer-valued inputs).
Inputs come from the seeded generators in ``workloads`` and are quantised by
the oracle on the CPU; full-size cases check sampled outputs.
"""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
import workloads
from oracle import e4m3_encode_rne, gemm_ref, gemm_ref_at, quant_act_ref, quant_weight_ref
from helpers import assert_gemm_close, bf16_rne, bf16_to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _gpu_gemm(a_q, a_s, w_q, w_s, path=None):
    args = [to_gpu(a_q), to_gpu(a_s), to_gpu(w_q), to_gpu(w_s)]
    c = fp8bq.gemm(*args) if path is None else fp8bq.gemm_forced(path, *args)
    torch.cuda.synchronize()
    return bf16_to_f64(c)


def _problem(m, n, k, outliers=True):
    a = workloads.activation(m, n, k, outliers=outliers)
    a_q, a_s = quant_act_ref(a)
    w_q, w_s = quant_weight_ref(workloads.weight(n, k))
    return a_q, a_s, w_q, w_s


def test_tiny_case():
    a, w = workloads.tiny_inputs()
    a_q, a_s = quant_act_ref(a)
    w_q, w_s = quant_weight_ref(w)
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what="tiny")


# Moderate sizes, whole output compared: several tiles, ragged M and N tails,
# both kernel paths.
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8, 9, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 127, 128, 129, 300])
@pytest.mark.parametrize("n,k", [(640, 1024), (700, 384)])
def test_moderate_sizes_whole_output(m, n, k):
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what=f"M={m} N={n} K={k}")


@pytest.mark.parametrize("n,k", [(16, 128), (17, 256), (1, 128), (130, 1152), (4100, 128)])
@pytest.mark.parametrize("m", [1, 7, 40, 70])
def test_odd_shapes(m, n, k):
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what=f"M={m} N={n} K={k}")


# Shapes that walk the streaming kernel's instance table: rows per workgroup
# -> 16-row tiles 1..5, K groups per wave 1..9, a K past the table (generic
# kernel), N not a multiple of 4, and workgroups whose last tile is short.
TABLE_SHAPES = [(1000, 9216), (12800, 1024), (20000, 2304), (4100, 5120), (5000, 9344), (300, 8704),
                (1026, 256), (7, 1280), (2999, 3072), (6000, 8704), (5120, 7168), (9000, 8704)]


@pytest.mark.parametrize("n,k", TABLE_SHAPES)
@pytest.mark.parametrize("m", [1, 3, 8, 16, 17, 32, 33, 48, 49, 64])
def test_streaming_instance_table(m, n, k):
    a = workloads.activation(m, n, k)
    a_q, a_s = quant_act_ref(a)
    w_q, w_s = quant_weight_ref(workloads.weight(n, k))
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    if n * k <= 12_000_000:
        assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what=f"M={m} N={n} K={k}")
    else:
        rng = np.random.default_rng([m, n, k])
        rows = rng.integers(0, m, 3000)
        cols = np.concatenate([rng.integers(0, n, 2000), np.arange(n - 1000, n)])
        ref = gemm_ref_at(a_q, a_s, w_q, w_s, rows, cols)
        assert_gemm_close(c[rows, cols], ref, what=f"M={m} N={n} K={k} (sampled)")


# 65..80 tokens stream with five 16-token sub-tiles where a workgroup has at
# most 2 row tiles and a wave at most 5 groups: every (tiles, groups) pair
# of that table, ragged N (not a multiple of 4, a short last tile), and the
# class's first, middle and last M.
WIDE_SHAPES = [(4000, 128), (3000, 2048), (4096, 3072), (1000, 4096), (2500, 5120),
               (5001, 384), (6000, 2560), (7000, 4096), (8190, 5120), (4100, 1152)]


@pytest.mark.parametrize("n,k", WIDE_SHAPES)
@pytest.mark.parametrize("m", [65, 72, 80])
def test_streaming_wide_token_class(m, n, k):
    assert fp8bq.lib().fp8bq_gemm_path(m, n, k) == fp8bq.PATH_STREAM
    a = workloads.activation(m, n, k)
    a_q, a_s = quant_act_ref(a)
    w_q, w_s = quant_weight_ref(workloads.weight(n, k))
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    if n * k <= 12_000_000:
        assert_gemm_close(c, gemm_ref(a_q, a_s, w_q, w_s), what=f"M={m} N={n} K={k}")
    else:
        rng = np.random.default_rng([m, n, k])
        rows = rng.integers(0, m, 3000)
        cols = np.concatenate([rng.integers(0, n, 2000), np.arange(n - 1000, n)])
        ref = gemm_ref_at(a_q, a_s, w_q, w_s, rows, cols)
        assert_gemm_close(c[rows, cols], ref, what=f"M={m} N={n} K={k} (sampled)")
    # the forced streaming path is the same single launch here
    c_forced = _gpu_gemm(a_q, a_s, w_q, w_s, path=fp8bq.PATH_STREAM)
    assert np.array_equal(c, c_forced)


def _integer_problem(m, n, k, vmax, scales, seed):
    rng = np.random.default_rng(seed)
    vals = np.arange(-vmax, vmax + 1, dtype=np.float32)
    a_q = e4m3_encode_rne(rng.choice(vals, size=(m, k)))
    w_q = e4m3_encode_rne(rng.choice(vals, size=(n, k)))
    sc = np.array(scales, np.float32)
    a_s = rng.choice(sc, size=(m, k // 128))
    w_s = rng.choice(sc, size=((n + 127) // 128, k // 128))
    return a_q, a_s, w_q, w_s


@pytest.mark.parametrize("m", [1, 2, 5, 8, 16, 32, 40, 64, 65, 80, 81, 200])
def test_integer_exact_bitwise_k1024(m):
    # |codes| <= 8, scales in {1/2, 1, 2}, K = 1024: every group sum, scaled
    # term and running sum is a multiple of 1/4 below 2^18, exact in fp32 in
    # any order, so C must equal bf16_rne(C_ref) bit for bit.
    a_q, a_s, w_q, w_s = _integer_problem(m, 768, 1024, 8, [0.5, 1.0, 2.0], seed=m)
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    want = bf16_rne(gemm_ref(a_q, a_s, w_q, w_s))
    assert np.array_equal(c, want)


@pytest.mark.parametrize("m", [1, 17, 24, 32])
def test_integer_exact_bitwise_k8704(m):
    # 68 groups: 9 per wave, where 17..32 tokens walk the chunks group-major
    # (and, past 2 row tiles, run the 64-token kernel); |codes| <= 2,
    # scales in {1, 2}: group sums < 2^10, running sums < 2^18, exact.
    for n in (5120, 9000):
        a_q, a_s, w_q, w_s = _integer_problem(m, n, 8704, 2, [1.0, 2.0], seed=200 + m)
        c = _gpu_gemm(a_q, a_s, w_q, w_s)
        want = bf16_rne(gemm_ref(a_q, a_s, w_q, w_s))
        assert np.array_equal(c, want), f"M={m} N={n}"


@pytest.mark.parametrize("m", [1, 3, 8, 64, 72, 130])
def test_integer_exact_bitwise_k5120(m):
    # |codes| <= 2, scales in {1, 2}, K = 5120 (40 groups split over waves):
    # group sums < 2^10, running sums < 2^17, all integers: exact in fp32.
    a_q, a_s, w_q, w_s = _integer_problem(m, 1024, 5120, 2, [1.0, 2.0], seed=100 + m)
    c = _gpu_gemm(a_q, a_s, w_q, w_s)
    want = bf16_rne(gemm_ref(a_q, a_s, w_q, w_s))
    assert np.array_equal(c, want)


@pytest.mark.parametrize("m", [1, 4, 8, 16, 33, 64, 65, 100, 128])
def test_stream_and_tiled_paths_agree(m):
    a_q, a_s, w_q, w_s = _problem(m, 1024, 2048)
    ref = gemm_ref(a_q, a_s, w_q, w_s)
    c_stream = _gpu_gemm(a_q, a_s, w_q, w_s, path=fp8bq.PATH_STREAM)
    c_tiled = _gpu_gemm(a_q, a_s, w_q, w_s, path=fp8bq.PATH_TILED)
    assert_gemm_close(c_stream, ref, what="stream")
    assert_gemm_close(c_tiled, ref, what="tiled")
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.max(np.abs(c_stream - c_tiled)) <= 2e-2 * rms + 2 ** -7 * np.max(np.abs(ref))


TILE_PATHS = (fp8bq.PATH_TILED_128x128, fp8bq.PATH_TILED_128x256, fp8bq.PATH_TILED_192x256,
              fp8bq.PATH_TILED_256x256, fp8bq.PATH_TILED_64x128, fp8bq.PATH_TILED_128x64,
              fp8bq.PATH_TILED_64x64)


# Every tile shape of the tiled kernel, whole output against the oracle on
# sizes with several tiles and ragged M and N tails (N not a multiple of 4
# takes the scalar store), and bitwise equality between the shapes: each
# output is summed group by group in the same order whatever the tiling.
@pytest.mark.parametrize("m,n,k", [(1, 300, 128), (65, 257, 1152), (300, 1040, 640), (517, 1100, 256)])
def test_tile_shapes_whole_output_and_bitwise(m, n, k):
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    ref = gemm_ref(a_q, a_s, w_q, w_s)
    args = [to_gpu(a_q), to_gpu(a_s), to_gpu(w_q), to_gpu(w_s)]
    outs = []
    for path in TILE_PATHS:
        c = fp8bq.gemm_forced(path, *args)
        torch.cuda.synchronize()
        assert_gemm_close(bf16_to_f64(c), ref, what=f"tile path {path} M={m} N={n} K={k}")
        outs.append(c)
    for path, c in zip(TILE_PATHS[1:], outs[1:]):
        assert torch.equal(c.view(torch.int16), outs[0].view(torch.int16)), f"tile path {path}"


# The tiled kernels copy the activation scales 8 groups at a time into a
# two-buffer array: K/128 = 13 and 17 groups end on a partly filled block of
# 8 (columns past the last group clamped), 17 also reuses the first buffer.
# Whole output against the oracle for the 8-wave tiles on their unclamped
# path (M >= BM, N a multiple of 256, the last token tile shifted back) and
# clamped path (N = 520), bitwise equal to 128 x 128 and 64 x 64 tiles.
@pytest.mark.parametrize("k", [13 * 128, 17 * 128])
@pytest.mark.parametrize("n", [512, 520])
def test_tiled_scale_blocks_partial_last(n, k):
    m = 300
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    ref = gemm_ref(a_q, a_s, w_q, w_s)
    args = [to_gpu(a_q), to_gpu(a_s), to_gpu(w_q), to_gpu(w_s)]
    outs = {}
    for path in (fp8bq.PATH_TILED_256x256, fp8bq.PATH_TILED_192x256, fp8bq.PATH_TILED_128x128,
                 fp8bq.PATH_TILED_64x64):
        outs[path] = fp8bq.gemm_forced(path, *args)
    torch.cuda.synchronize()
    for path, c in outs.items():
        assert_gemm_close(bf16_to_f64(c), ref, what=f"tile path {path} N={n} K={k}")
        assert torch.equal(c.view(torch.int16), outs[fp8bq.PATH_TILED_128x128].view(torch.int16)), f"tile path {path}"


# Grids of the 8-wave tiles with a last round of at most 128 tiles run that
# round as column halves (a second launch of BM x BN/2 workgroups): whole
# output against the oracle and bitwise equal to 128 x 128 tiles, for the
# exact (N a multiple of BN) and the clamped kernel, including a column half
# wholly past N (N = 8000: the last 256-column tile's second half starts at
# 8064).
@pytest.mark.parametrize("m,n,k,path", [(2000, 8000, 256, fp8bq.PATH_TILED_192x256),
                                        (2100, 8000, 256, fp8bq.PATH_TILED_256x256),
                                        (2000, 8192, 256, fp8bq.PATH_TILED_192x256),
                                        (2100, 8192, 384, fp8bq.PATH_TILED_256x256)])
def test_tiled2_last_round_column_halves(m, n, k, path):
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    ref = gemm_ref(a_q, a_s, w_q, w_s)
    args = [to_gpu(a_q), to_gpu(a_s), to_gpu(w_q), to_gpu(w_s)]
    c = fp8bq.gemm_forced(path, *args)
    c_128 = fp8bq.gemm_forced(fp8bq.PATH_TILED_128x128, *args)
    torch.cuda.synchronize()
    assert_gemm_close(bf16_to_f64(c), ref, what=f"tile path {path} M={m} N={n} K={k}")
    assert torch.equal(c.view(torch.int16), c_128.view(torch.int16))


def test_deterministic_repeat_calls():
    a_q, a_s, w_q, w_s = _problem(8, 5120, 3072)
    args = [to_gpu(a_q), to_gpu(a_s), to_gpu(w_q), to_gpu(w_s)]
    c1 = fp8bq.gemm(*args).clone()
    c2 = fp8bq.gemm(*args).clone()
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_k_zero_writes_zeros_and_m_zero_is_noop():
    dev = torch.device("cuda")
    out = torch.full((3, 5), 7.0, dtype=torch.bfloat16, device=dev)
    fp8bq.gemm(torch.zeros((3, 0), dtype=torch.uint8, device=dev), torch.zeros((3, 0), device=dev),
               torch.zeros((5, 0), dtype=torch.uint8, device=dev), torch.zeros((1, 0), device=dev), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    c = fp8bq.gemm(torch.zeros((0, 128), dtype=torch.uint8, device=dev), torch.zeros((0, 1), device=dev),
                   torch.zeros((5, 128), dtype=torch.uint8, device=dev), torch.zeros((1, 1), device=dev))
    assert c.shape == (0, 5)


# Full sizes of the five logged shapes, the launch configuration the
# benchmark times: A and W are quantised on the GPU (bit-exactness of that
# step is checked here on the rows and row blocks that are sampled), and the
# oracle recomputes sampled outputs from its own quantisation of the same
# seeded rows.
def _full_cases():
    cases = []
    for n, k in workloads.SHAPES:  # grouped by shape: one weight upload each
        # every shape: decode, verify, the concurrent batches 16 / 32 / 64
        ms = [1, 8, 16, 32, 64]
        if (n, k) == (5120, 3072):
            # both token classes of the 2-tile, 3-groups-per-wave instances
            # (9..16 and 17..32), and 64 x 128 tiles at 256
            ms = [1, 8, 9, 12, 16, 17, 24, 32, 64, 65, 80, 256]
        if (n, k) == (8192, 5120):
            ms = [1, 8, 16, 32, 64, 80, 192]  # 128 x 64 tiles at 192
        if (n, k) == (17408, 5120):
            ms = list(range(1, 9)) + [16, 32, 40, 48, 64]
        if (n, k) == (5120, 8704):
            ms = [1, 8, 16, 17, 32, 64, 65, 128]
        if (n, k) == (7168, 5120):
            ms = [1, 8, 16, 32, 64, 65, 100]
        if (n, k) in workloads.PREFILL_SHAPES:
            ms.append(workloads.PREFILL_M)
        cases += [(m, n, k) for m in ms]
    return cases


FULL_CASES = _full_cases()


@pytest.fixture(scope="module")
def weights_on_gpu():
    cache = {}

    def get(n, k):
        if (n, k) not in cache:
            cache.clear()  # one full-size weight resident at a time
            w_q, w_s = fp8bq.quant_weight(to_gpu(workloads.weight(n, k)))
            cache[(n, k)] = (w_q, w_s)
        return cache[(n, k)]

    return get


@pytest.mark.parametrize("m,n,k", FULL_CASES, ids=[f"M{m}-N{n}-K{k}" for m, n, k in FULL_CASES])
def test_full_size_sampled_outputs(m, n, k, weights_on_gpu):
    w_q, w_s = weights_on_gpu(n, k)
    a = workloads.activation(m, n, k)
    a_q, a_s = fp8bq.quant_act(to_gpu(a))
    c = fp8bq.gemm(a_q, a_s, w_q, w_s)
    torch.cuda.synchronize()

    rng = np.random.default_rng([m, n, k])
    nb = (n + 127) // 128
    blocks = sorted({0, nb - 1, int(rng.integers(0, nb)), int(rng.integers(0, nb))})
    rows = sorted({0, m - 1, *rng.integers(0, m, size=min(m, 6)).tolist()})
    # oracle quantisation of the sampled weight row blocks and token rows
    a_rows = a[rows]
    oa_q, oa_s = quant_act_ref(a_rows)
    assert np.array_equal(a_q[rows].cpu().numpy(), oa_q)
    assert np.array_equal(a_s[rows].cpu().numpy().view(np.uint32), oa_s.view(np.uint32))
    ow = [quant_weight_ref(workloads.weight_block(n, k, b)) for b in blocks]
    for b, (oq, os_) in zip(blocks, ow):
        assert np.array_equal(w_q[128 * b : 128 * b + 128].cpu().numpy(), oq), f"W codes, block row {b}"
        assert np.array_equal(w_s[b : b + 1].cpu().numpy().view(np.uint32), os_.view(np.uint32))
    # sampled outputs: every sampled token row against 64 columns of each block
    wq_cat = np.concatenate([oq for oq, _ in ow])
    ws_cat = np.concatenate([os_ for _, os_ in ow])  # one scale row per sampled block
    col_local = np.concatenate([128 * i + rng.choice(oq.shape[0], size=min(64, oq.shape[0]), replace=False)
                                for i, (oq, _) in enumerate(ow)])
    col_global = np.concatenate([128 * b + (col_local[(col_local >= 128 * i) & (col_local < 128 * i + 128)] - 128 * i)
                                 for i, b in enumerate(blocks)])
    rr, cc = np.meshgrid(np.arange(len(rows)), np.arange(len(col_local)), indexing="ij")
    ref = gemm_ref_at(oa_q, oa_s, wq_cat, ws_cat, rr.ravel(), col_local[cc.ravel()])
    got = bf16_to_f64(c[rows][:, torch.from_numpy(col_global).to(c.device)]).ravel()
    assert_gemm_close(got, ref, what=f"M={m} N={n} K={k}")


# The prefill size on both prefill shapes: the tile shape gemm() picks
# (256 x 256 and 192 x 256 tiles there), whose sampled outputs are checked
# against the oracle above, is bitwise equal to every other tile shape.
@pytest.mark.parametrize("n,k", workloads.PREFILL_SHAPES)
def test_prefill_tile_shapes_bitwise(n, k, weights_on_gpu):
    w_q, w_s = weights_on_gpu(n, k)
    m = workloads.PREFILL_M
    a_q, a_s = fp8bq.quant_act(to_gpu(workloads.activation(m, n, k)))
    c = fp8bq.gemm(a_q, a_s, w_q, w_s)
    for path in TILE_PATHS:
        c_path = fp8bq.gemm_forced(path, a_q, a_s, w_q, w_s)
        torch.cuda.synchronize()
        assert torch.equal(c_path.view(torch.int16), c.view(torch.int16)), f"tile path {path}"
