"""Shared helpers for the GPU parity tests (no method arithmetic here)."""

import numpy as np
import torch

# GEMM acceptance bound: |C_gpu - C_ref| <= 1e-2 * rms(C_ref) + 2^-8 * |C_ref|
# elementwise. The second term is one bf16 rounding (unit roundoff 2^-8);
# the first absorbs fp32 accumulation in an order other than the oracle's.
RMS_TOL = 1e-2
BF16_U = 2.0 ** -8


def device():
    return torch.device("cuda:0")


def to_gpu(x, dtype=None):
    t = x if isinstance(x, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().to(device())


def bf16_to_f64(c: torch.Tensor) -> np.ndarray:
    return c.detach().to("cpu").to(torch.float64).numpy()


def assert_gemm_close(c_gpu: np.ndarray, c_ref: np.ndarray, rms=None, what=""):
    """Check the acceptance bound; return max|err| / rms for reporting."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    assert c_gpu.shape == c_ref.shape
    assert np.all(np.isfinite(c_gpu)), what
    if rms is None:
        rms = float(np.sqrt(np.mean(c_ref ** 2))) if c_ref.size else 0.0
    err = np.abs(c_gpu - c_ref)
    bound = RMS_TOL * rms + BF16_U * np.abs(c_ref)
    bad = err > bound
    if np.any(bad):
        i = np.argmax(err - bound)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} outputs out of bound; worst at flat index {i}: "
            f"gpu={c_gpu.flat[i]!r} ref={c_ref.flat[i]!r} bound={bound.flat[i]!r} rms={rms!r}")
    return float(err.max() / rms) if rms > 0 and err.size else 0.0


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 values exactly representable in fp32 -> bf16 (RNE) -> fp64."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)), "not fp32-exact"
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
