"""Seeded synthetic inputs for the block-FP8 decode GEMM.

This module only draws random numbers and rounds them to the input dtypes;
it contains none of the quantisation or GEMM arithmetic. Both the CPU oracle
tests and the HIP-path tests and benchmark take their inputs from here.

The pages measure real Qwen3.8-27B-FP8 weights on ShareGPT prompts (page 1,
section "test background"), a 3,465-token prompt (page 2, section 4.2) and
256-token prompts (page 3, section 2.3). None of that data is available, and
the GEMM's cost does not depend on the values, so Gaussian stand-ins with the
pages' shapes replace them:

* weights: W = 0.02 * N(0, 1) in fp32, shape [N, K];
* activations: A = N(0, 1), with 0.1 % of the entries (at least one, at
  uniformly drawn distinct positions) multiplied by 20 as outliers, rounded
  to bf16 (round-to-nearest-even via torch);
* the tiny case (M=1, N=512, K=1024) uses one generator seeded 0, drawing W
  first and then A, with no outliers.

Two-stage vocabulary scoring (page 1, section "single-stream optimisation")
runs the same GEMM against a vocabulary-sized projection. The pages print
neither the vocabulary size nor the survivor count: V = 152064 (a
Qwen-family vocabulary padded to a multiple of 128) and k = 64 stand in.
Its inputs are the hidden state (an activation of width K = 5120), the
projection W (drawn like any weight, bf16 copy by RNE) and, for the
selection and rescoring stages alone, seeded logits and survivor indices.

Seeds: W for shape (N, K) is drawn one 128-row block at a time, block b
from ``numpy.random.default_rng([0, N, K, b])`` (so a test can rebuild any
row block without drawing the whole matrix); A for (M, N, K) comes from
``default_rng([1, N, K, M])``, normals first, outlier positions second.
"""

import numpy as np
import torch

# The five (N, K) shapes logged in page 2 (ownding.com L20 report), section 8.
SHAPES = [(17408, 5120), (5120, 3072), (5120, 8704), (7168, 5120), (8192, 5120)]
TINY = (1, 512, 1024)  # (M, N, K)
PREFILL_M = 3465  # prompt length of page 2's output test (section 4.2)
PREFILL_SHAPES = [(17408, 5120), (5120, 8704)]
VOCAB = 152064  # stand-in vocabulary size
SURVIVORS = 64  # stand-in survivor count
HIDDEN = 5120
OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 20.0


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 CPU tensor, round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def tiny_inputs():
    """(A bf16 [1, 1024], W fp32 [512, 1024]) of the tiny case, seed 0."""
    m, n, k = TINY
    rng = np.random.default_rng(0)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    a = rng.standard_normal((m, k)).astype(np.float32)
    return to_bf16(a), w


def weight_block(n: int, k: int, b: int) -> np.ndarray:
    """Rows 128 b .. min(128 b + 128, N) - 1 of weight(n, k)."""
    rows = min(128, n - 128 * b)
    if rows <= 0:
        raise ValueError(f"row block {b} is outside N={n}")
    rng = np.random.default_rng([0, n, k, b])
    return (np.float32(0.02) * rng.standard_normal((rows, k), dtype=np.float32)).astype(np.float32)


def weight(n: int, k: int) -> np.ndarray:
    """W fp32 [N, K] = 0.02 * N(0, 1), drawn per 128-row block."""
    out = np.empty((n, k), dtype=np.float32)
    for b in range((n + 127) // 128):
        out[128 * b : 128 * b + 128] = weight_block(n, k, b)
    return out


def activation(m: int, n: int, k: int, outliers: bool = True) -> torch.Tensor:
    """A bf16 [M, K] = N(0, 1) with 0.1 % outliers x20, seeded by (N, K, M)."""
    rng = np.random.default_rng([1, n, k, m])
    a = rng.standard_normal((m, k), dtype=np.float32)
    if outliers and m * k > 0:
        count = max(1, int(round(OUTLIER_FRACTION * m * k)))
        idx = rng.choice(m * k, size=count, replace=False)
        flat = a.reshape(-1)
        flat[idx] = flat[idx] * np.float32(OUTLIER_FACTOR)
    return to_bf16(a)


def random_codes(shape, seed: int) -> np.ndarray:
    """Uniform e4m3fn codes over all 254 finite codes (NaN codes excluded)."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = c + (c >= 0x7F)  # skip 0x7F; 0xFF is never drawn
    return c.astype(np.uint8)


def random_scales(shape, seed: int, lo: float = 2.0 ** -12, hi: float = 2.0 ** -4) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [lo, hi)."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float32)


def logit_bits(m: int, v: int, kind: str, seed: int) -> np.ndarray:
    """bf16 bit patterns uint16 [M, V] for the selection stage.

    kind "normal": bf16 of 3 N(0, 1) (bf16's 8-bit mantissa makes equal
    values common); "ties": 5 distinct values, mostly equal; "bits": every
    16-bit pattern equally likely (signed zeros, infinities, NaN patterns)."""
    rng = np.random.default_rng([2, m, v, seed])
    if kind == "normal":
        x = (3.0 * rng.standard_normal((m, v))).astype(np.float32)
        return to_bf16(x).view(torch.int16).numpy().view(np.uint16)
    if kind == "ties":
        vals = np.array([-1.5, -0.0, 0.0, 0.75, 2.0], dtype=np.float32)
        return to_bf16(rng.choice(vals, size=(m, v))).view(torch.int16).numpy().view(np.uint16)
    if kind == "bits":
        return rng.integers(0, 1 << 16, size=(m, v), dtype=np.int64).astype(np.uint16)
    raise ValueError(kind)


def survivor_indices(m: int, v: int, k: int, seed: int) -> np.ndarray:
    """int32 [M, k]: per row, k distinct vocabulary indices in random order."""
    rng = np.random.default_rng([3, m, v, k, seed])
    return np.stack([rng.choice(v, size=k, replace=False) for _ in range(m)]).astype(np.int32)
