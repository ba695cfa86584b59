"""Weight-only block-FP8 GEMM (W8A16) reference in fp64 (test infrastructure
only).

Page 1 (SmartX blog, "Qwen3.8-27B performance optimisation"), section
"single-stream optimisation", contrasts the W8A8 backend, which quantises the
activation on every call, with a W8A16 backend that keeps the activation in
16-bit floats and only the weight in FP8, and reports the latter faster at a
single stream. With the same block-FP8 weights (e4m3fn codes, one fp32 scale
per 128 x 128 block) and a bf16 activation, the output is

    C[m, n] = sum_g  sw[n // 128, g] * sum_{k in group g} A[m, k] * dec(Wq[n, k])

Each product of a bf16 value (8 significant bits) and an e4m3 value (4) is
exact in fp64; the group sums and the scaled sum over groups round in fp64
only, so the result is correct to a few fp64 ulps of sum |terms|.
"""

import numpy as np

from .e4m3 import e4m3_decode

GROUP = 128


def _check(a, w_q, w_s):
    a = np.asarray(a, dtype=np.float64)
    w_q = np.asarray(w_q, dtype=np.uint8)
    w_s = np.asarray(w_s, dtype=np.float32)
    m, k = a.shape
    n, k2 = w_q.shape
    if k != k2 or k % GROUP:
        raise ValueError(f"gemm_w8a16_ref: K mismatch or K % 128 != 0 ({k}, {k2})")
    g = k // GROUP
    if w_s.shape != (-(-n // GROUP), g):
        raise ValueError(f"gemm_w8a16_ref: bad weight scale shape {w_s.shape}")
    return a, w_q, w_s, m, n, k, g


def gemm_w8a16_ref(a, w_q, w_s) -> np.ndarray:
    """Whole [M, N] output in fp64; `a` holds the bf16 activation values
    (any float array whose entries are bf16 numbers)."""
    a, w_q, w_s, m, n, k, g = _check(a, w_q, w_s)
    w_dec = e4m3_decode(w_q)  # [N, K] float64, exact
    sw_rows = np.repeat(w_s.astype(np.float64), GROUP, axis=0)[:n]  # [N, G]
    c = np.zeros((m, n), dtype=np.float64)
    for gi in range(g):
        ks = slice(gi * GROUP, (gi + 1) * GROUP)
        c += (a[:, ks] @ w_dec[:, ks].T) * sw_rows[None, :, gi]
    return c


def gemm_w8a16_ref_at(a, w_q, w_s, rows, cols) -> np.ndarray:
    """C[rows[i], cols[i]] for sampled output positions, fp64, same formula."""
    a, w_q, w_s, m, n, k, g = _check(a, w_q, w_s)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a_g = a[rows].reshape(len(rows), g, GROUP)
    w_dec = e4m3_decode(w_q[cols]).reshape(len(cols), g, GROUP)
    partial = np.sum(a_g * w_dec, axis=2)  # [P, G]
    return np.sum(w_s[cols // GROUP].astype(np.float64) * partial, axis=1)
