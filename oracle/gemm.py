"""Block-scaled FP8 GEMM reference in fp64 (test infrastructure only).

The layer is y = x W^T with W stored as "W8A8 Block FP8" of shape (N, K)
(page 2, ownding.com L20 report, section 8, the five logged N, K shapes).
With the activation quantised per token per 128-wide group and the weight
per 128 x 128 block, the output is

    C[m, n] = sum_g  sa[m, g] * sw[n // 128, g]
                     * sum_{k in group g} dec(Aq[m, k]) * dec(Wq[n, k])

Every fp8 x fp8 product has at most 8 significant bits and is a multiple of
2^-18 below 2^18, so each 128-term group sum is exact in fp64; the product
of two fp32 scales is exact in fp64. The only roundings are the final fp64
scale-times-group-sum products and the sum over groups, so the result is
correct to a few fp64 ulps of sum |terms|.
"""

import numpy as np

from .e4m3 import e4m3_decode

GROUP = 128


def _check(a_q, a_s, w_q, w_s):
    a_q = np.asarray(a_q, dtype=np.uint8)
    w_q = np.asarray(w_q, dtype=np.uint8)
    a_s = np.asarray(a_s, dtype=np.float32)
    w_s = np.asarray(w_s, dtype=np.float32)
    m, k = a_q.shape
    n, k2 = w_q.shape
    if k != k2 or k % GROUP:
        raise ValueError(f"gemm_ref: K mismatch or K % 128 != 0 ({k}, {k2})")
    g = k // GROUP
    if a_s.shape != (m, g) or w_s.shape != (-(-n // GROUP), g):
        raise ValueError(f"gemm_ref: bad scale shapes {a_s.shape} {w_s.shape}")
    return a_q, a_s, w_q, w_s, m, n, k, g


def gemm_ref(a_q, a_s, w_q, w_s) -> np.ndarray:
    """Whole [M, N] output in fp64, one 128-wide K group at a time."""
    a_q, a_s, w_q, w_s, m, n, k, g = _check(a_q, a_s, w_q, w_s)
    a_dec = e4m3_decode(a_q)  # [M, K] float64, exact
    w_dec = e4m3_decode(w_q)  # [N, K] float64, exact
    sw_rows = np.repeat(w_s.astype(np.float64), GROUP, axis=0)[:n]  # [N, G]
    c = np.zeros((m, n), dtype=np.float64)
    for gi in range(g):
        ks = slice(gi * GROUP, (gi + 1) * GROUP)
        partial = a_dec[:, ks] @ w_dec[:, ks].T  # exact group sums
        scale = a_s[:, gi].astype(np.float64)[:, None] * sw_rows[None, :, gi]
        c += scale * partial
    return c


def gemm_ref_at(a_q, a_s, w_q, w_s, rows, cols) -> np.ndarray:
    """C[rows[i], cols[i]] for sampled output positions, fp64, same formula."""
    a_q, a_s, w_q, w_s, m, n, k, g = _check(a_q, a_s, w_q, w_s)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a_dec = e4m3_decode(a_q[rows]).reshape(len(rows), g, GROUP)
    w_dec = e4m3_decode(w_q[cols]).reshape(len(cols), g, GROUP)
    partial = np.sum(a_dec * w_dec, axis=2)  # [P, G], exact group sums
    scale = a_s[rows].astype(np.float64) * w_s[cols // GROUP].astype(np.float64)
    return np.sum(scale * partial, axis=1)
