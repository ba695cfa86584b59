"""The C-ABI library loads, exports what include/fp8bq.h declares, and
rejects bad arguments on the host before touching any device (CPU only)."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bq.h")


@pytest.fixture(scope="module")
def fp8bq():
    import memory_bound_w8a8_amd as m

    if not os.path.exists(m.LIB_PATH):
        from memory_bound_w8a8_amd import build

        build.build()
    return m


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:int|int64_t|const char \*)\s*(fp8bq_\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_abi():
    assert _declared() == {"fp8bq_quant_act", "fp8bq_quant_weight", "fp8bq_gemm", "fp8bq_gemm_path",
                           "fp8bq_gemm_forced", "fp8bq_gemm_workspace_bytes", "fp8bq_gemm_ws", "fp8bq_gemm_ws_forced", "fp8bq_gemm_tile_shape", "fp8bq_gemm_fused", "fp8bq_gemm_w8a16",
                           "fp8bq_topk_workspace_bytes",
                           "fp8bq_topk_bf16", "fp8bq_topk_bf16_noalloc", "fp8bq_rescore_bf16", "fp8bq_mb_read", "fp8bq_mb_empty",
                           "fp8bq_mb_mfma_e4m3", "fp8bq_mb_mfma_e4m3_data", "fp8bq_mb_mfma_e4m3_scaled",
                           "fp8bq_status_string"}


def test_library_exports_every_declared_symbol(fp8bq):
    raw = ctypes.CDLL(fp8bq.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(fp8bq.EXPORTS) == _declared()


def test_status_strings(fp8bq):
    L = fp8bq.lib()
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = L.fp8bq_status_string(st).decode()
        assert s and s != "unknown status"
    assert L.fp8bq_status_string(42).decode() == "unknown status"


FAKE = 1 << 20  # an aligned, never-dereferenced address for host-side checks


def test_gemm_shape_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_gemm(-1, 4, 128, p, p, p, p, p, None) == -2
    assert L.fp8bq_gemm(1, -4, 128, p, p, p, p, p, None) == -2
    assert L.fp8bq_gemm(1, 4, -128, p, p, p, p, p, None) == -2
    assert L.fp8bq_gemm(1, 4, 100, p, p, p, p, p, None) == -2
    assert L.fp8bq_gemm(1 << 21, 1 << 21, 128, p, p, p, p, p, None) == -2  # M*N > 2^40
    assert L.fp8bq_gemm_forced(1, 129, 4, 128, p, p, p, p, p, None) == -2  # stream path serves M <= 128
    assert L.fp8bq_gemm_forced(10, 1, 4, 128, p, p, p, p, p, None) == -2  # unknown path
    assert L.fp8bq_gemm_forced(-1, 1, 4, 128, p, p, p, p, p, None) == -2


def test_gemm_quick_return_and_null_and_alignment(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_gemm(0, 4, 128, None, None, None, None, None, None) == 0
    assert L.fp8bq_gemm(4, 0, 128, None, None, None, None, None, None) == 0
    assert L.fp8bq_gemm(1, 4, 128, None, p, p, p, p, None) == -1
    assert L.fp8bq_gemm(1, 4, 128, p, None, p, p, p, None) == -1
    assert L.fp8bq_gemm(1, 4, 128, p, p, None, p, p, None) == -1
    assert L.fp8bq_gemm(1, 4, 128, p, p, p, None, p, None) == -1
    assert L.fp8bq_gemm(1, 4, 128, p, p, p, p, None, None) == -1
    assert L.fp8bq_gemm(1, 4, 128, p + 8, p, p, p, p, None) == -3
    assert L.fp8bq_gemm(1, 4, 128, p, p + 2, p, p, p, None) == -3
    assert L.fp8bq_gemm(1, 4, 128, p, p, p + 1, p, p, None) == -3
    assert L.fp8bq_gemm(1, 4, 128, p, p, p, p + 1, p, None) == -3
    assert L.fp8bq_gemm(1, 4, 128, p, p, p, p, p + 2, None) == -3


def test_quant_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_quant_act(-1, 128, p, p, p, None) == -2
    assert L.fp8bq_quant_act(1, 130, p, p, p, None) == -2
    assert L.fp8bq_quant_act(0, 128, None, None, None, None) == 0
    assert L.fp8bq_quant_act(1, 128, None, p, p, None) == -1
    assert L.fp8bq_quant_act(1, 128, p + 2, p, p, None) == -3
    assert L.fp8bq_quant_act(1, 128, p, p + 4, p, None) == -3
    assert L.fp8bq_quant_act(1, 128, p, p, p + 1, None) == -3
    assert L.fp8bq_quant_weight(1, 64, p, p, p, None) == -2
    assert L.fp8bq_quant_weight(128 * 70000, 128, p, p, p, None) == -2
    assert L.fp8bq_quant_weight(0, 128, None, None, None, None) == 0
    assert L.fp8bq_quant_weight(5, 128, p, None, p, None) == -1
    assert L.fp8bq_quant_weight(5, 128, p + 4, p, p, None) == -3


def test_w8a16_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_gemm_w8a16(-1, 4, 128, p, p, p, p, None) == -2
    assert L.fp8bq_gemm_w8a16(1, 4, 100, p, p, p, p, None) == -2
    assert L.fp8bq_gemm_w8a16(17, 4, 128, p, p, p, p, None) == -2  # one 16-token tile at most
    assert L.fp8bq_gemm_w8a16(1, 4, 9216 + 128, p, p, p, p, None) == -2  # past 72 groups
    assert L.fp8bq_gemm_w8a16(0, 4, 128, None, None, None, None, None) == 0
    assert L.fp8bq_gemm_w8a16(1, 0, 128, None, None, None, None, None) == 0
    assert L.fp8bq_gemm_w8a16(1, 4, 128, None, p, p, p, None) == -1
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, None, p, p, None) == -1
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p, None, p, None) == -1
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p, p, None, None) == -1
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p + 2, p, p, p, None) == -3
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p + 8, p, p, None) == -3
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p, p + 1, p, None) == -3
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p, p, p + 2, None) == -3


def test_fused_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_gemm_fused(-1, 4, 128, p, p, p, p, None) == -2
    assert L.fp8bq_gemm_fused(1, 4, 100, p, p, p, p, None) == -2
    assert L.fp8bq_gemm_fused(9, 4, 128, p, p, p, p, None) == -2  # up to 8 tokens
    assert L.fp8bq_gemm_fused(1, 4, 9216 + 128, p, p, p, p, None) == -2
    assert L.fp8bq_gemm_fused(0, 4, 128, None, None, None, None, None) == 0
    assert L.fp8bq_gemm_fused(1, 4, 128, None, p, p, p, None) == -1
    assert L.fp8bq_gemm_fused(1, 4, 128, p, p, p, None, None) == -1
    assert L.fp8bq_gemm_fused(1, 4, 128, p + 2, p, p, p, None) == -3
    assert L.fp8bq_gemm_fused(1, 4, 128, p, p, p + 1, p, None) == -3


def test_topk_workspace_size(fp8bq):
    L = fp8bq.lib()
    # first level: one list of k per G chunks of 1024 logits (G = min(4,
    # 1024 // k)); second: at most one per 1024 // k lists; 8 bytes an entry
    for m, v, k in ((1, 152064, 64), (4, 152064, 50), (3, 4096, 256), (2, 4097, 1), (1, 10, 10), (16, 1 << 20, 7),
                    (2, 300000, 100)):
        g = min(4, 1024 // k)
        l1 = -(-(-(-v // 1024)) // g)
        l2 = -(-l1 // (1024 // k))
        assert L.fp8bq_topk_workspace_bytes(m, v, k) == (l1 + l2) * m * k * 8, (m, v, k)
    assert L.fp8bq_topk_workspace_bytes(0, 100, 5) == 8 * 0
    assert L.fp8bq_topk_workspace_bytes(1, 100, 0) == -2
    assert L.fp8bq_topk_workspace_bytes(1, 100, 257) == -2
    assert L.fp8bq_topk_workspace_bytes(1, 100, 101) == -2
    assert L.fp8bq_topk_workspace_bytes(-1, 100, 5) == -2
    assert L.fp8bq_topk_workspace_bytes(1, 1 << 31, 5) == -2


def test_topk_noalloc_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    f = L.fp8bq_topk_bf16_noalloc
    scratch = fp8bq.TOPK_SCRATCH_BYTES
    assert scratch == 4 << 20
    # largest M whose workspace fits the 4 MiB scratch at V = 152064, k = 64
    per_row = L.fp8bq_topk_workspace_bytes(1, 152064, 64)
    assert per_row * 199 <= scratch < per_row * 200
    assert f(200, 152064, 64, p, p, p, None) == -6  # too large for the scratch array
    assert f(2, 1000, 0, p, p, p, None) == -2
    assert f(2, 1000, 257, p, p, p, None) == -2
    assert f(2, 7, 8, p, p, p, None) == -2
    assert f(-1, 1000, 8, p, p, p, None) == -2
    assert f(0, 1000, 8, None, None, None, None) == 0
    assert f(2, 1000, 8, None, p, p, None) == -1
    assert f(2, 1000, 8, p, None, p, None) == -1
    assert f(2, 1000, 8, p, p, None, None) == -1
    assert f(2, 1000, 8, p + 2, p, p, None) == -3
    assert f(2, 1000, 8, p, p + 2, p, None) == -3
    assert f(2, 1000, 8, p, p, p + 2, None) == -3


def test_topk_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    ws = L.fp8bq_topk_workspace_bytes(2, 1000, 8)
    assert L.fp8bq_topk_bf16(2, 1000, 0, p, p, ws, p, p, None) == -2
    assert L.fp8bq_topk_bf16(2, 1000, 257, p, p, ws, p, p, None) == -2
    assert L.fp8bq_topk_bf16(2, 7, 8, p, p, ws, p, p, None) == -2  # k > V
    assert L.fp8bq_topk_bf16(-1, 1000, 8, p, p, ws, p, p, None) == -2
    assert L.fp8bq_topk_bf16(2, 1 << 31, 8, p, p, ws, p, p, None) == -2
    assert L.fp8bq_topk_bf16(1 << 11, 1 << 24, 8, p, p, 1 << 40, p, p, None) == -2  # 2^22 workgroups
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p, ws - 1, p, p, None) == -2
    assert L.fp8bq_topk_bf16(0, 1000, 8, None, None, 0, None, None, None) == 0
    assert L.fp8bq_topk_bf16(2, 1000, 8, None, p, ws, p, p, None) == -1
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, None, ws, p, p, None) == -1
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p, ws, None, p, None) == -1
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p, ws, p, None, None) == -1
    assert L.fp8bq_topk_bf16(2, 1000, 8, p + 2, p, ws, p, p, None) == -3
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p + 8, ws, p, p, None) == -3
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p, ws, p + 2, p, None) == -3
    assert L.fp8bq_topk_bf16(2, 1000, 8, p, p, ws, p, p + 2, None) == -3


def test_rescore_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_rescore_bf16(1, 64, 100, 0, p, p, p, p, p, None) == -2  # k < 1
    assert L.fp8bq_rescore_bf16(1, 60, 100, 4, p, p, p, p, p, None) == -2  # K % 8
    assert L.fp8bq_rescore_bf16(-1, 64, 100, 4, p, p, p, p, p, None) == -2
    assert L.fp8bq_rescore_bf16(1, 64, 1 << 31, 4, p, p, p, p, p, None) == -2
    assert L.fp8bq_rescore_bf16(1 << 22, 64, 100, 4, p, p, p, p, p, None) == -2  # too many rows
    assert L.fp8bq_rescore_bf16(0, 64, 100, 4, None, None, None, None, None, None) == 0
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, None, p, p, p, p, None) == -1
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, None, p, p, p, None) == -1
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, None, p, p, None) == -1
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p, None, p, None) == -1
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p, p, None, None) == -1
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p + 8, p, p, p, p, None) == -3
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p + 8, p, p, p, None) == -3
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p + 2, p, p, None) == -3
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p, p + 2, p, None) == -3
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p, p, p + 2, None) == -3


def test_gemm_workspace_plan(fp8bq):
    # host-only: the K-split plan of fp8bq_gemm_ws (split x M x N x 4 bytes)
    L = fp8bq.lib()
    assert L.fp8bq_gemm_workspace_bytes(0, 17408, 5120) == 0
    assert L.fp8bq_gemm_workspace_bytes(64, 17408, 5120) == 0  # streamed, no tiles
    assert L.fp8bq_gemm_workspace_bytes(65, 17408, 5120) % (65 * 17408 * 4) == 0
    for n, k in ((17408, 5120), (5120, 3072), (5120, 8704), (7168, 5120), (8192, 5120)):
        splits = []
        for m in (81, 96, 128):
            b = L.fp8bq_gemm_workspace_bytes(m, n, k)
            assert b >= 0 and b % (4 * m * n) == 0 and b // (4 * m * n) <= 64, (m, n, k, b)
            splits.append(b // (4 * m * n))
        # few tiles: some of these token counts split, except where the 24
        # groups of K = 3072 leave too little K per part
        assert (max(splits) >= 2) == (k > 3072), (n, k, splits)
        for m in range(1, 33, 3):
            assert L.fp8bq_gemm_workspace_bytes(m, n, k) == 0
        # 33..64 tokens split only where the streaming waves walk 8..9 groups
        # over at most 2 row tiles (K = 8704 here)
        for m in (33, 48, 64):
            assert (L.fp8bq_gemm_workspace_bytes(m, n, k) > 0) == (k == 8704), (m, n, k)
    # a prefill-sized grid fills the CUs without splitting
    assert L.fp8bq_gemm_workspace_bytes(3465, 17408, 5120) == 0
    assert L.fp8bq_gemm_workspace_bytes(100, 4096, 128) == 0  # one group: nothing to split
    assert L.fp8bq_gemm_workspace_bytes(-1, 4, 128) == -2
    assert L.fp8bq_gemm_workspace_bytes(1, 4, 100) == -2


def test_gemm_ws_argument_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    # the workspace: negative size, NULL with a size, misaligned
    assert L.fp8bq_gemm_ws(100, 4096, 1024, p, p, p, p, p, p, -1, None) == -2
    assert L.fp8bq_gemm_ws(100, 4096, 1024, p, p, p, p, p, None, 64, None) == -1
    assert L.fp8bq_gemm_ws(100, 4096, 1024, p, p, p, p, p, p + 8, 64, None) == -3
    # the GEMM's own checks come first
    assert L.fp8bq_gemm_ws(100, 4096, 1000, p, p, p, p, p, p, 64, None) == -2
    assert L.fp8bq_gemm_ws(100, 4096, 1024, None, p, p, p, p, p, 64, None) == -1
    assert L.fp8bq_gemm_ws(0, 4096, 1024, p, p, p, p, p, None, 0, None) == 0
    # forced plans: only the gemm_tiled_kernel shapes split, 2..min(64, K/128) parts, enough workspace
    big = 64 * 100 * 4096 * 4
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_192x256, 2, 100, 4096, 1024, p, p, p, p, p, p, big, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_256x256, 2, 100, 4096, 1024, p, p, p, p, p, p, big, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_STREAM, 2, 100, 4096, 1024, p, p, p, p, p, p, big, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_128x128, 9, 100, 4096, 1024, p, p, p, p, p, p, big, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_128x128, 0, 100, 4096, 1024, p, p, p, p, p, p, big, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_128x128, 65, 100, 4096, 65 * 128, p, p, p, p, p, p, big,
                                  None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_64x64, 3, 100, 4096, 1024, p, p, p, p, p, p,
                                  3 * 100 * 4096 * 4 - 1, None) == -2
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_64x64, 3, 100, 4096, 1024, p, p, p, p, p, None, 64, None) == -1
    # a grid of 2^31 or more workgroups: (2^20 / 64)^2 tiles of 64 x 64 in 8 parts
    big_mn = 1 << 20
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_64x64, 8, big_mn, big_mn, 1024, p, p, p, p, p, p, 1 << 62,
                                  None) == -2


def test_gemm_path_dispatch_by_explicit_m_ranges(fp8bq):
    L = fp8bq.lib()
    assert L.fp8bq_gemm_path(0, 17408, 5120) == fp8bq.PATH_NONE
    for m in list(range(1, 65)):
        assert L.fp8bq_gemm_path(m, 17408, 5120) == fp8bq.PATH_STREAM, m
    for m in (65, 128, 2048, 3465, 4096):
        assert L.fp8bq_gemm_path(m, 17408, 5120) == fp8bq.PATH_TILED, m
    # 65..80 tokens stream where one round of 256 workgroups covers N with
    # at most 32 rows each (N <= 8192) and a wave holds at most 5 of the
    # K/128 groups (K <= 5120); otherwise, and beyond 80, the tiled kernel
    for n, k in ((5120, 3072), (7168, 5120), (8192, 5120), (128, 1024), (8192, 128)):
        for m in (65, 72, 80):
            assert L.fp8bq_gemm_path(m, n, k) == fp8bq.PATH_STREAM, (m, n, k)
        for m in (81, 100, 128, 129, 3465):
            assert L.fp8bq_gemm_path(m, n, k) == fp8bq.PATH_TILED, (m, n, k)
    for n, k in ((5120, 8704), (17408, 5120), (8193, 5120), (8192, 5248), (16256, 5120)):
        for m in (65, 80, 81, 128):
            assert L.fp8bq_gemm_path(m, n, k) == fp8bq.PATH_TILED, (m, n, k)
    assert L.fp8bq_gemm_path(1, 17408, 5000) == -2


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error; a GPU is present")
def test_device_error_without_gpu(fp8bq):
    # All arguments valid: the only failure left is the device check, which
    # must come back as an error rather than a launch.
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_gemm(1, 4, 128, p, p, p, p, p, None) == -4
    assert L.fp8bq_gemm_ws(1, 4, 128, p, p, p, p, p, None, 0, None) == -4
    assert L.fp8bq_gemm_ws_forced(fp8bq.PATH_TILED_64x64, 2, 100, 4096, 1024, p, p, p, p, p, p,
                                  2 * 100 * 4096 * 4, None) == -4
    assert L.fp8bq_quant_act(1, 128, p, p, p, None) == -4
    assert L.fp8bq_gemm_w8a16(1, 4, 128, p, p, p, p, None) == -4
    assert L.fp8bq_gemm_fused(1, 4, 128, p, p, p, p, None) == -4
    assert L.fp8bq_topk_bf16(1, 100, 5, p, p, L.fp8bq_topk_workspace_bytes(1, 100, 5), p, p, None) == -4
    assert L.fp8bq_rescore_bf16(1, 64, 100, 4, p, p, p, p, p, None) == -4


def test_binding_rejects_cpu_tensors(fp8bq):
    with pytest.raises(ValueError):
        fp8bq.quant_act(torch.zeros(1, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fp8bq.gemm(torch.zeros(1, 128, dtype=torch.uint8), torch.zeros(1, 1), torch.zeros(4, 128, dtype=torch.uint8),
                   torch.zeros(1, 1))


def test_measurement_kernel_argument_errors(fp8bq):
    L = fp8bq.lib()
    p = FAKE
    assert L.fp8bq_mb_read(p, 24, 256, p, None) == -2  # bytes % 16
    assert L.fp8bq_mb_read(p, -16, 256, p, None) == -2
    assert L.fp8bq_mb_read(p, 16, 0, p, None) == -2  # grid
    assert L.fp8bq_mb_read(p, 16, 65537, p, None) == -2
    assert L.fp8bq_mb_read(None, 16, 256, p, None) == -1  # NULL allowed only for bytes == 0
    assert L.fp8bq_mb_read(p, 16, 256, None, None) == -1
    assert L.fp8bq_mb_read(p + 8, 16, 256, p, None) == -3
    assert L.fp8bq_mb_empty(0, 64, None) == -2
    assert L.fp8bq_mb_empty(1, 100, None) == -2  # block not a multiple of 64
    assert L.fp8bq_mb_empty(1, 2048, None) == -2
    assert L.fp8bq_mb_mfma_e4m3(0, 1, 0x38, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3(1, -1, 0x38, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3(1, 1, 0x7F, p, None) == -2  # NaN code
    assert L.fp8bq_mb_mfma_e4m3(1, 1, 0xFF, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3(1, 1, 256, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3(1, 1, 0x38, None, None) == -1
    assert L.fp8bq_mb_mfma_e4m3(1, 1, 0x38, p + 2, None) == -3
    assert L.fp8bq_mb_mfma_e4m3_data(0, 1, p, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_data(65537, 1, p, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_data(1, -1, p, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_data(1, 1, None, p, None) == -1
    assert L.fp8bq_mb_mfma_e4m3_data(1, 1, p, None, None) == -1
    assert L.fp8bq_mb_mfma_e4m3_data(1, 1, p + 8, p, None) == -3
    assert L.fp8bq_mb_mfma_e4m3_data(1, 1, p, p + 2, None) == -3
    assert L.fp8bq_mb_mfma_e4m3_scaled(0, 1, p, 1.0, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_scaled(65537, 1, p, 1.0, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, -1, p, 1.0, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, 1 << 25, p, 1.0, p, None) == -2
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, 1, None, 1.0, p, None) == -1
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, 1, p, 1.0, None, None) == -1
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, 1, p + 8, 1.0, p, None) == -3
    assert L.fp8bq_mb_mfma_e4m3_scaled(1, 1, p, 1.0, p + 2, None) == -3


def test_tile_shape_rule_takes_the_measured_choices(fp8bq):
    """The tiled kernel's shape rule (least grid rounds x measured step
    cost) on points where the shapes were timed side by side (each
    expectation is the shape that measured fastest there), then its
    tie-break and its range."""
    L = fp8bq.lib()
    shape = lambda m, n, k: fp8bq.PATH_NAMES[L.fp8bq_gemm_tile_shape(m, n, k)]
    assert shape(3465, 17408, 5120) == "tiled 256x256"  # 952 tiles, 4 rounds
    assert shape(3465, 5120, 8704) == "tiled 192x256"  # 380 tiles, 2 rounds (256 x 256: 280, 1.09)
    assert shape(2048, 5120, 3072) == "tiled 192x256"
    assert shape(4096, 7168, 5120) == "tiled 256x256"
    assert shape(1024, 8192, 5120) == "tiled 128x256"
    assert shape(1024, 17408, 5120) == "tiled 192x256"
    assert shape(3072, 17408, 5120) == "tiled 256x256"  # 274 us against 301 for 192 x 256
    assert shape(4096, 17408, 5120) == "tiled 256x256"  # 355 against 376
    assert shape(2048, 17408, 5120) == "tiled 192x256"  # 180 against 195
    assert shape(2560, 5120, 8704) == "tiled 256x256"
    for m in (65, 96, 128):
        assert shape(m, 17408, 5120) == "tiled 128x128", m  # 136 tiles; smaller ones overflow a round
        for n, k in ((5120, 3072), (5120, 8704), (7168, 5120), (8192, 5120)):
            assert shape(m, n, k) == "tiled 64x64", (m, n)  # 160..256 tiles, one round
    assert shape(192, 17408, 5120) == "tiled 64x128"
    assert shape(192, 5120, 8704) == "tiled 64x64"
    assert shape(192, 7168, 5120) == "tiled 128x64"
    assert shape(192, 8192, 5120) == "tiled 128x64"
    assert shape(256, 5120, 8704) == "tiled 64x128"  # equal cost to 128 x 64, equal tiles: first in order
    # every answer is a shape fp8bq_gemm_forced accepts; sizes as for the GEMM
    for m in (1, 64, 65, 300, 3465, 100000):
        for n in (1, 127, 5120, 17408, 152064):
            assert fp8bq.PATH_TILED_128x128 <= L.fp8bq_gemm_tile_shape(m, n, 5120) <= fp8bq.PATH_TILED_64x64
    assert L.fp8bq_gemm_tile_shape(0, 5120, 5120) == fp8bq.PATH_NONE
    assert L.fp8bq_gemm_tile_shape(1, 5120, 100) == -2
    assert L.fp8bq_gemm_tile_shape(-1, 5120, 128) == -2
