"""Two-stage vocabulary scoring (test infrastructure only).

Page 1 (SmartX blog, "Qwen3.8-27B performance optimisation"), section
"single-stream optimisation": the draft head reads the whole vocabulary
projection every step, and a two-stage scheme cuts that traffic -- score all
candidates coarsely in FP8, then score the survivors exactly in BF16 -- while
keeping the low-precision scores from hurting draft acceptance. The pages
give neither the vocabulary size nor how many candidates survive; here the
stages are:

1. coarse logits: the block-FP8 GEMM of the (quantised) hidden state with the
   FP8 copy of the vocabulary projection, as `gemm.gemm_ref`;
2. `topk_ref`: the k largest coarse logits of each row;
3. `rescore_ref`: exact dot products of the hidden state with the BF16 rows
   of the survivors; the best survivor is the row's pick.

Order used by top-k and by the final pick (the pages are silent): values are
bf16 numbers compared by their bit key (sign-magnitude mapped to a monotone
unsigned order, so -0 ranks just below +0), equal keys by lower index.
"""

import numpy as np


def bf16_key(bits: np.ndarray) -> np.ndarray:
    """Monotone unsigned 16-bit key of bf16 bit patterns: larger key = larger
    value (negative patterns are inverted, positive ones get the top bit)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000).astype(np.uint32)


def topk_ref(logit_bits: np.ndarray, k: int):
    """Per row, the k entries with the largest bf16 key, ties to the lower
    index, listed in that order. `logit_bits` holds bf16 bit patterns
    (uint16 [M, V]). Returns (indices int64 [M, k], bit patterns uint16)."""
    bits = np.asarray(logit_bits, dtype=np.uint16)
    m, v = bits.shape
    if not 1 <= k <= v:
        raise ValueError(f"topk_ref: k={k} outside 1..{v}")
    key = bf16_key(bits)
    idx = np.empty((m, k), dtype=np.int64)
    for i in range(m):
        order = np.lexsort((np.arange(v), -key[i].astype(np.int64)))  # key desc, index asc
        idx[i] = order[:k]
    return idx, np.take_along_axis(bits, idx, axis=1)


def rescore_ref(h: np.ndarray, w: np.ndarray, idx: np.ndarray):
    """Exact scores of the survivors in fp64: s[m, j] = sum_k h[m, k] *
    w[idx[m, j], k], with h and w the bf16 values as floats; and each row's
    pick, the survivor with the largest score (ties to the lower index).
    Returns (scores float64 [M, k], pick int64 [M])."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    scores = np.einsum("mk,mjk->mj", h, w[idx])
    pick = np.empty(idx.shape[0], dtype=np.int64)
    for i in range(idx.shape[0]):
        best = max(range(idx.shape[1]), key=lambda j: (scores[i, j], -idx[i, j]))
        pick[i] = idx[i, best]
    return scores, pick
