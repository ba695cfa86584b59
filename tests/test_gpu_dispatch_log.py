"""The kernel-choice log (FP8BQ_LOG=1): each distinct (entry point, M, N,
K) decision is printed once, naming the instance the shape's M range and
(N, K) select. Runs one child process (the variable is read once per
process)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

CHILD = r"""
import torch
import memory_bound_w8a8_amd as fp8bq
dev = torch.device("cuda:0")
k = 5120
w_q, w_s = fp8bq.quant_weight(torch.randn(17408, k, device=dev) * 0.02)
for m in (1, 3, 1, 16, 32, 64, 65, 3465):
    a_q, a_s = fp8bq.quant_act(torch.randn(m, k, device=dev).to(torch.bfloat16))
    fp8bq.gemm(a_q, a_s, w_q, w_s)
fp8bq.gemm_fused(torch.randn(2, k, device=dev).to(torch.bfloat16), w_q, w_s)
# 65..80 tokens stream where a workgroup has 2 row tiles and a wave 5 groups
w_q, w_s = fp8bq.quant_weight(torch.randn(8192, k, device=dev) * 0.02)
for m in (80, 81):
    a_q, a_s = fp8bq.quant_act(torch.randn(m, k, device=dev).to(torch.bfloat16))
    fp8bq.gemm(a_q, a_s, w_q, w_s)
# with a workspace, 65..~256 tokens split K where the cost model says so
w_q, w_s = fp8bq.quant_weight(torch.randn(5120, 8704, device=dev) * 0.02)
a_q, a_s = fp8bq.quant_act(torch.randn(96, 8704, device=dev).to(torch.bfloat16))
fp8bq.gemm_ws(a_q, a_s, w_q, w_s)
# tile shapes by rounds x step cost on (5120, 8704): 192 x 256 at the prefill size,
# 128 x 256 where it keeps the grid within the same rounds
w_q, w_s = fp8bq.quant_weight(torch.randn(5120, 8704, device=dev) * 0.02)
for m in (3465, 1024, 128, 192, 256):
    a_q, a_s = fp8bq.quant_act(torch.randn(m, 8704, device=dev).to(torch.bfloat16))
    fp8bq.gemm(a_q, a_s, w_q, w_s)
torch.cuda.synchronize()
"""


def test_dispatch_log_names_each_decision_once():
    env = dict(os.environ, FP8BQ_LOG="1", PYTHONPATH=ROOT)
    proc = subprocess.run([sys.executable, "-c", CHILD], env=env, cwd=ROOT, capture_output=True, text=True,
                          timeout=300)
    assert proc.returncode == 0, proc.stderr[-2000:]
    lines = [ln for ln in proc.stderr.splitlines() if ln.startswith("fp8bq: ")]
    assert len(lines) == len(set(lines))  # M = 1 twice: logged once
    got = {ln.split(" -> ")[0]: ln.split(" -> ")[1] for ln in lines}
    assert got["fp8bq: gemm(stream) M=1 N=17408 K=5120"].startswith("gemm_rows_kernel MT=16 act=codes TILES=5 GMAX=5")
    assert "rows/wg=68 grid=256" in got["fp8bq: gemm(stream) M=3 N=17408 K=5120"]
    assert got["fp8bq: gemm(stream) M=16 N=17408 K=5120"].startswith("gemm_rows_kernel MT=16 act=lines")
    assert got["fp8bq: gemm(stream) M=32 N=17408 K=5120"].startswith("gemm_rows_kernel MT=32 act=lines")
    assert got["fp8bq: gemm(stream) M=64 N=17408 K=5120"].startswith("gemm_rows64_kernel")
    assert got["fp8bq: gemm(tiled) M=65 N=17408 K=5120"].startswith("gemm_tiled_kernel BM=128 BN=128")
    assert got["fp8bq: gemm(tiled) M=3465 N=17408 K=5120"].startswith("gemm_tiled2_kernel BM=256 BN=256 8 waves 2 stages grid=952")
    assert got["fp8bq: gemm(stream) M=80 N=8192 K=5120"] == (
        "gemm_rows64_kernel MS=5 TILES=2 GMAX=5 rows/wg=32 grid=256")
    assert got["fp8bq: gemm(tiled) M=81 N=8192 K=5120"].startswith("gemm_tiled")
    ws_line = got["fp8bq: gemm(tiled, split K) M=96 N=5120 K=8704"]
    assert ws_line.startswith("gemm_tiled_kernel BM=") and " parts) + split_reduce_kernel" in ws_line
    assert got["fp8bq: gemm_fused M=2 N=17408 K=5120"].startswith("gemm_rows_kernel MT=16 act=bf16 TOK=2")
    # 380 tiles of 192 x 256 (one round, then the last 124 tiles as 248 column halves in about half a
    # round) beat 280 of 256 x 256 (one round + 48 halves) and 560 of 128 x 256 (2.19 rounds)
    assert got["fp8bq: gemm(tiled) M=3465 N=5120 K=8704"] == (
        "gemm_tiled2_kernel BM=192 BN=256 8 waves 2 stages grid=380 (256 whole + 248 column halves)")
    # 160 tiles of 128 x 256 fit one round; the larger tiles cost more per step
    assert got["fp8bq: gemm(tiled) M=1024 N=5120 K=8704"] == "gemm_tiled_kernel BM=128 BN=256 8 waves 3 stages grid=160"
    # few tokens on a narrow weight: 64 x 64 tiles fill the CUs while their
    # grid fits one round (160 at M = 128, 240 at 192); at 256 tokens (320)
    # the 4-wave halves do (160 tiles of 64 x 128, the first of the two in order)
    assert got["fp8bq: gemm(tiled) M=128 N=5120 K=8704"] == "gemm_tiled_kernel BM=64 BN=64 4 waves 3 stages grid=160"
    assert got["fp8bq: gemm(tiled) M=192 N=5120 K=8704"] == "gemm_tiled_kernel BM=64 BN=64 4 waves 3 stages grid=240"
    assert got["fp8bq: gemm(tiled) M=256 N=5120 K=8704"] == "gemm_tiled_kernel BM=64 BN=128 4 waves 3 stages grid=160"
