"""Block-FP8 quantisers (test infrastructure only; see the package header).

Activation side: page 1 (SmartX blog), section "single-stream optimisation",
states that the W8A8 FP8 backend quantises the activation of each linear
layer on every call (Marlin skips it). Page 2, section 8, names the layer
"W8A8 Block FP8". The group shape (one scale per token per 128 consecutive K
entries), the scale rule s = amax / 448 in fp32 and the weight block shape
(128 x 128) are the DeepSeek-style block-FP8 scheme the pages' tuning script
targets; the pages do not spell them out.

Readings of points the pages leave open (listed again in the design notes):

* quantise by IEEE fp32 division x / s, not by multiplying with 448 / amax;
* a group whose amax is 0 gets s = 1.0 (codes are then signed zeros);
* clamp x / s to [-448, 448] before rounding, so no NaN code is produced;
* round to e4m3fn nearest-even, keep the sign of zero.

All arithmetic below is numpy float32, which is IEEE binary32 with
round-to-nearest-even and gradual underflow, i.e. exactly the fp32
operations a GPU performs with correctly rounded division.
"""

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode_rne

GROUP = 128


def _as_float32(x) -> np.ndarray:
    """Accept a numpy array or a CPU torch tensor; return float32 numpy."""
    if hasattr(x, "detach"):  # torch tensor (bf16 or fp32), widened exactly
        import torch

        x = x.detach().to("cpu").to(torch.float32).numpy()
    return np.asarray(x, dtype=np.float32)


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    """s = amax / 448 in fp32 (IEEE division), or 1.0 for an all-zero group."""
    amax = amax.astype(np.float32)
    s = np.divide(amax, np.float32(E4M3_MAX), dtype=np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def _encode_scaled(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """codes = e4m3_rne(clamp(x / s, -448, 448)), all in fp32."""
    q = np.divide(x, s, dtype=np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode_rne(q)


def quant_act_ref(a):
    """Per-token 1x128-group activation quantisation.

    a: [M, K] activations (bf16 values; a torch bf16 tensor or float32 numpy
       holding bf16-representable values). K must be a multiple of 128.
    Returns (codes uint8 [M, K], scales float32 [M, K / 128]) with, for every
    token m and group g:
        x    = a[m, 128 g : 128 g + 128] in fp32 (exact widening of bf16)
        amax = max |x|
        s    = fp32(amax / 448), or 1.0 when amax == 0
        code = e4m3_rne(clamp(fp32(x / s), -448, 448))
    """
    x = _as_float32(a)
    if x.ndim != 2 or x.shape[1] % GROUP != 0:
        raise ValueError(f"quant_act_ref: need [M, K] with K % 128 == 0, got {x.shape}")
    m, k = x.shape
    groups = x.reshape(m, k // GROUP, GROUP)
    amax = np.max(np.abs(groups), axis=2) if m > 0 else np.zeros((0, k // GROUP), np.float32)
    s = _scale_from_amax(amax)
    codes = _encode_scaled(groups, s[:, :, None]).reshape(m, k)
    return codes, s


def quant_weight_ref(w):
    """Per-128x128-block weight quantisation.

    w: [N, K] float32 weights; K a multiple of 128, N arbitrary (the last row
       block may hold fewer than 128 rows).
    Returns (codes uint8 [N, K], scales float32 [ceil(N / 128), K / 128]);
    block (b, g) covers rows 128 b .. min(128 b + 128, N) - 1 and columns
    128 g .. 128 g + 127, and is quantised exactly like one activation group
    but with the amax taken over the whole block.
    """
    x = _as_float32(w)
    if x.ndim != 2 or x.shape[1] % GROUP != 0:
        raise ValueError(f"quant_weight_ref: need [N, K] with K % 128 == 0, got {x.shape}")
    n, k = x.shape
    nb, kg = -(-n // GROUP), k // GROUP
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty((nb, kg), dtype=np.float32)
    for b in range(nb):
        rows = x[b * GROUP : min((b + 1) * GROUP, n)]
        blocks = rows.reshape(rows.shape[0], kg, GROUP)
        amax = np.max(np.abs(blocks), axis=(0, 2))
        s = _scale_from_amax(amax)
        scales[b] = s
        codes[b * GROUP : b * GROUP + rows.shape[0]] = _encode_scaled(blocks, s[None, :, None]).reshape(rows.shape[0], k)
    return codes, scales
