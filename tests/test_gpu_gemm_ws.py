"""GPU parity of fp8bq_gemm_ws, the block-FP8 GEMM with a caller workspace
whose K-split plan spreads each tile's K/128 groups over several
workgroups (fp32 partial tiles, summed in a fixed order by a second
launch), against the fp64 oracle.

Acceptance as for fp8bq_gemm: |C_gpu - C_ref| <= 1e-2 * rms(C_ref) +
2^-8 * |C_ref| (fp32 accumulation in any order plus one bf16 rounding);
bit-exact bf16 where every partial sum is exact in fp32; identical calls
give identical bits; without enough workspace the call is fp8bq_gemm,
bit for bit.
"""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
import workloads
from oracle import e4m3_encode_rne, gemm_ref, gemm_ref_at, quant_act_ref, quant_weight_ref
from helpers import assert_gemm_close, bf16_rne, bf16_to_f64, to_gpu

pytestmark = pytest.mark.gpu

SPLIT_PATHS = (fp8bq.PATH_TILED_128x128, fp8bq.PATH_TILED_128x256, fp8bq.PATH_TILED_64x128,
               fp8bq.PATH_TILED_128x64, fp8bq.PATH_TILED_64x64)


def _problem(m, n, k):
    a_q, a_s = quant_act_ref(workloads.activation(m, n, k))
    w_q, w_s = quant_weight_ref(workloads.weight(n, k))
    return a_q, a_s, w_q, w_s


# Every tile shape that splits, K parts of unequal length (9 groups in 2, 4
# and 7 parts), ragged M and N (partial token and weight tiles); N = 701
# makes M x N odd, which takes the partial tiles' and the reduction's
# one-output-at-a-time paths.
@pytest.mark.parametrize("path", SPLIT_PATHS)
@pytest.mark.parametrize("split", [2, 4, 7])
@pytest.mark.parametrize("n", [700, 701])
def test_forced_split_whole_output_and_repeatable(path, split, n):
    m, k = 70, 1152
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    args = [to_gpu(x) for x in (a_q, a_s, w_q, w_s)]
    c = fp8bq.gemm_ws_forced(path, split, *args)
    c2 = fp8bq.gemm_ws_forced(path, split, *args)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    assert_gemm_close(bf16_to_f64(c), gemm_ref(a_q, a_s, w_q, w_s), what=f"path {path} split {split} N {n}")


# More parts than the reduction's compile-time instances (up to 16): the
# generic any-count path, 40 groups in 20 and 40 parts.
@pytest.mark.parametrize("split", [20, 40])
def test_forced_split_many_parts(split):
    m, n, k = 65, 640, 5120
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    args = [to_gpu(x) for x in (a_q, a_s, w_q, w_s)]
    c = fp8bq.gemm_ws_forced(fp8bq.PATH_TILED_64x64, split, *args)
    torch.cuda.synchronize()
    assert_gemm_close(bf16_to_f64(c), gemm_ref(a_q, a_s, w_q, w_s), what=f"split {split}")


# |codes| <= 8, scales in {1/2, 1, 2}, K = 1024: every product, group sum,
# partial tile and their sum is a multiple of 1/4 below 2^18, exact in fp32
# in any order, so every split gives bf16_rne(C_ref) bit for bit.
@pytest.mark.parametrize("split", [2, 3, 8])
def test_split_integer_exact_bitwise(split):
    rng = np.random.default_rng(300 + split)
    m, n, k = 100, 768, 1024
    vals = np.arange(-8, 9, dtype=np.float32)
    a_q = e4m3_encode_rne(rng.choice(vals, size=(m, k)))
    w_q = e4m3_encode_rne(rng.choice(vals, size=(n, k)))
    sc = np.array([0.5, 1.0, 2.0], np.float32)
    a_s = rng.choice(sc, size=(m, k // 128))
    w_s = rng.choice(sc, size=((n + 127) // 128, k // 128))
    want = bf16_rne(gemm_ref(a_q, a_s, w_q, w_s))
    args = [to_gpu(x) for x in (a_q, a_s, w_q, w_s)]
    for path in SPLIT_PATHS:
        c = fp8bq.gemm_ws_forced(path, split, *args)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_to_f64(c), want), f"path {path}"


def test_without_enough_workspace_it_is_the_plain_gemm():
    m, n, k = 100, 1024, 8704
    need = fp8bq.gemm_workspace_bytes(m, n, k)
    assert need > 0
    a_q, a_s, w_q, w_s = [to_gpu(x) for x in _problem(m, n, k)]
    c = fp8bq.gemm(a_q, a_s, w_q, w_s)
    small = torch.empty(need - 16, dtype=torch.uint8, device=a_q.device)
    c_small = fp8bq.gemm_ws(a_q, a_s, w_q, w_s, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(c_small.view(torch.int16), c.view(torch.int16))
    # up to 32 tokens there is no split plan and no workspace is read
    assert fp8bq.gemm_workspace_bytes(32, n, k) == 0
    c32 = fp8bq.gemm_ws(a_q[:32], a_s[:32], w_q, w_s)
    torch.cuda.synchronize()
    assert torch.equal(c32.view(torch.int16), fp8bq.gemm(a_q[:32], a_s[:32], w_q, w_s).view(torch.int16))


# The default plan at the logged shapes' full sizes, 65..256 tokens (the
# counts whose tiles leave CUs idle) and 33..64 on (5120, 8704), where the
# split replaces streaming: A and W quantised on the GPU (checked
# bit for bit against the oracle on the sampled rows and row blocks), then
# sampled outputs against the oracle.
WS_CASES = [(m, n, k) for n, k in workloads.SHAPES for m in (65, 80, 96, 128, 200, 256)]
WS_CASES += [(m, 5120, 8704) for m in (33, 48, 64)]  # deep K: the split replaces streaming


@pytest.fixture(scope="module")
def weights_on_gpu():
    cache = {}

    def get(n, k):
        if (n, k) not in cache:
            cache.clear()
            cache[(n, k)] = fp8bq.quant_weight(to_gpu(workloads.weight(n, k)))
        return cache[(n, k)]

    return get


@pytest.mark.parametrize("m,n,k", WS_CASES, ids=[f"M{m}-N{n}-K{k}" for m, n, k in WS_CASES])
def test_default_plan_full_size_sampled(m, n, k, weights_on_gpu):
    w_q, w_s = weights_on_gpu(n, k)
    a = workloads.activation(m, n, k)
    a_q, a_s = fp8bq.quant_act(to_gpu(a))
    c = fp8bq.gemm_ws(a_q, a_s, w_q, w_s)
    c2 = fp8bq.gemm_ws(a_q, a_s, w_q, w_s)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))

    rng = np.random.default_rng([m, n, k, 7])
    nb = (n + 127) // 128
    blocks = sorted({0, nb - 1, int(rng.integers(0, nb))})
    rows = sorted({0, m - 1, *rng.integers(0, m, size=6).tolist()})
    oa_q, oa_s = quant_act_ref(a[rows])
    assert np.array_equal(a_q[rows].cpu().numpy(), oa_q)
    ow = [quant_weight_ref(workloads.weight_block(n, k, b)) for b in blocks]
    for b, (oq, os_) in zip(blocks, ow):
        assert np.array_equal(w_q[128 * b : 128 * b + 128].cpu().numpy(), oq), f"W codes, block row {b}"
    wq_cat = np.concatenate([oq for oq, _ in ow])
    ws_cat = np.concatenate([os_ for _, os_ in ow])
    col_local = np.concatenate([128 * i + rng.choice(oq.shape[0], size=min(64, oq.shape[0]), replace=False)
                                for i, (oq, _) in enumerate(ow)])
    col_global = np.concatenate([128 * b + (col_local[(col_local >= 128 * i) & (col_local < 128 * i + 128)] - 128 * i)
                                 for i, b in enumerate(blocks)])
    rr, cc = np.meshgrid(np.arange(len(rows)), np.arange(len(col_local)), indexing="ij")
    ref = gemm_ref_at(oa_q, oa_s, wq_cat, ws_cat, rr.ravel(), col_local[cc.ravel()])
    got = bf16_to_f64(c[rows][:, torch.from_numpy(col_global).to(c.device)]).ravel()
    assert_gemm_close(got, ref, what=f"M={m} N={n} K={k} (split plan, workspace "
                                     f"{fp8bq.gemm_workspace_bytes(m, n, k)} B)")


# The workspace's contents are arbitrary on entry: a workspace full of 0xff
# bytes (NaN partial tiles) gives the same bits as a zeroed one, twice in a
# row, with partial token and weight tiles, so no element of the workspace
# is read before this call wrote it.
@pytest.mark.parametrize("path, split", [(fp8bq.PATH_TILED_128x256, 3), (fp8bq.PATH_TILED_64x64, 5)])
def test_forced_split_any_workspace_contents(path, split):
    m, n, k = 65, 1000, 1280
    a_q, a_s, w_q, w_s = _problem(m, n, k)
    args = [to_gpu(x) for x in (a_q, a_s, w_q, w_s)]
    need = split * m * n * 4
    zeroed = torch.zeros(need, dtype=torch.uint8, device="cuda")
    dirty = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    c0 = fp8bq.gemm_ws_forced(path, split, *args, workspace=zeroed)
    c1 = fp8bq.gemm_ws_forced(path, split, *args, workspace=dirty)
    c2 = fp8bq.gemm_ws_forced(path, split, *args, workspace=dirty)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))
    assert torch.equal(c0.view(torch.int16), c2.view(torch.int16))
    assert_gemm_close(bf16_to_f64(c0), gemm_ref(a_q, a_s, w_q, w_s), what=f"path {path} split {split}")
