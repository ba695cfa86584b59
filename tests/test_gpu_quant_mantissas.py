"""GPU parity of the in-kernel quotient over every bf16 amax mantissa.

The quantisation kernels form x / s from a reciprocal and one fma
correction (fp8bq_quant_act) or from a two-term reciprocal (the quantisation
inside fp8bq_gemm_fused), with the IEEE division only below amax = 2^-96,
so bit-exactness depends on the (x, amax) pair. These tests take every one of the 128 mantissa
patterns of the group maximum at 29 exponent fields -- bf16 subnormal
maxima, maxima whose scale amax / 448 is an fp32 subnormal, the 2^-104 ..
2^-96 neighbourhood of the switch to division, and normal maxima up to the
largest binade -- and, for each maximum a, every bf16 x with
a * 2^-19 <= |x| <= a of both signs (everything that quantises to a non-zero
code, and the first values that round to zero).

* fp8bq_quant_act: codes and scales bit-exact against quant_act_ref.
* fp8bq_gemm_fused, every quantisation layout (1, 2, 3..4 and 5..8
  tokens): against an identity weight (N = K, code 1.0 on the diagonal) the
  GEMM definition reduces to C[m, n] = dec(q[m, n]) * s[m, g] * sw[g, g]
  (g = n / 128), with one fp32 rounding of that exact product (the kernel's
  scale fma) and one bf16 rounding. The weight scale sw[g, g] is a power of
  two chosen per block so that every product is an fp32 normal number, and
  all tokens of a block share their maximum's binade. A code one step off
  changes C by at least 1/16 relative, far more than the bf16 rounding, so
  C equal to the value computed from the oracle's codes and scales means
  equal codes. (Signed zero is invisible through the GEMM: the -0 of
  quant_act is checked above.)
"""

import functools

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
from oracle import e4m3_decode, quant_act_ref
from helpers import bf16_rne, to_gpu

pytestmark = pytest.mark.gpu

# bf16 exponent fields of the maxima: 0 = subnormal maxima; <= 10: the scale
# amax / 448 is an fp32 subnormal; 23..31: 2^-104 .. 2^-96; then normal
# binades across the range up to the largest.
EXPONENT_FIELDS = (0, 1, 2, 9, 10, 11, 12, 20, 22, 23, 24, 25, 29, 30, 31, 32, 33, 40, 64, 100, 120, 126, 127,
                   128, 135, 136, 160, 200, 254)


@functools.lru_cache(maxsize=1)
def _mantissa_band():
    """(groups uint16 [G, 128] of bf16 patterns, owner int64 [G]: index of the
    group's maximum in `maxima`, maxima uint16 [A]). Each group holds its
    maximum at position 0 and 127 values below it (the last group of a
    maximum padded with zeros)."""
    pos = np.arange(1, 0x7F80, dtype=np.uint32)  # positive finite bf16 patterns
    vals = (pos << 16).view(np.float32)
    groups, owner, maxima = [], [], []
    for e in EXPONENT_FIELDS:
        for mant in range(128):
            p = (e << 7) | mant
            if p == 0:
                continue
            a = np.float32((np.uint32(p) << 16).view(np.float32))
            sel = pos[(vals <= a) & (vals >= a * np.float32(2.0 ** -19))]
            xs = np.concatenate([sel, sel | 0x8000]).astype(np.uint16)
            n_g = -(-xs.size // 127)
            body = np.zeros(n_g * 127, dtype=np.uint16)
            body[: xs.size] = xs
            g = np.empty((n_g, 128), dtype=np.uint16)
            g[:, 0] = p
            g[:, 1:] = body.reshape(n_g, 127)
            groups.append(g)
            owner.append(np.full(n_g, len(maxima), dtype=np.int64))
            maxima.append(p)
    return np.concatenate(groups), np.concatenate(owner), np.array(maxima, dtype=np.uint16)


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@functools.lru_cache(maxsize=1)
def _oracle_band():
    groups, _, _ = _mantissa_band()
    q, s = quant_act_ref(_bf16(groups))  # one token per group: [G, 128], [G, 1]
    return q, s[:, 0]


def test_quant_act_every_amax_mantissa():
    groups, _, _ = _mantissa_band()
    rows = -(-groups.shape[0] // 64)
    padded = np.zeros((rows * 64, 128), dtype=np.uint16)
    padded[: groups.shape[0]] = groups
    a = _bf16(padded.reshape(rows, 64 * 128))
    a_q, a_s = fp8bq.quant_act(to_gpu(a))
    torch.cuda.synchronize()
    got_q = a_q.cpu().numpy().reshape(rows * 64, 128)[: groups.shape[0]]
    got_s = a_s.cpu().numpy().reshape(rows * 64)[: groups.shape[0]]
    want_q, want_s = _oracle_band()
    bad = np.nonzero(np.any(got_q != want_q, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} groups with code mismatches; first: max pattern {groups[bad[0], 0]:#06x}, "
                           f"x patterns {groups[bad[0]][got_q[bad[0]] != want_q[bad[0]]][:8]}")
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "scale bits differ"


K_ID = 8192  # 64 groups per token; N = K for the identity weight
BLOCKS = K_ID // 128


def _block_scale_exponent(amax_bits: np.ndarray) -> np.ndarray:
    """Power of two per maximum that brings s * 2^e near 2^-8: every product
    dec(code) * s * 2^e is then an fp32 normal number. Kept within fp32
    normal powers of two."""
    a = (amax_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _, ex = np.frexp(a)  # a = f 2^ex, f in [0.5, 1)
    return np.clip(1 - ex, -100, 127)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_fused_every_amax_mantissa_identity_weight(m):
    groups, owner, maxima = _mantissa_band()
    oq, os_ = _oracle_band()
    exps = _block_scale_exponent(maxima)
    # blocks: M groups of one maximum each (a maximum's last block repeats its
    # first groups); calls: 64 blocks each (the last call repeats block 0)
    block_groups = []
    for ai in range(maxima.size):
        gi = np.nonzero(owner == ai)[0]
        need = -(-gi.size // m) * m
        gi = np.resize(gi, need)
        block_groups.append(gi.reshape(-1, m))
    block_groups = np.concatenate(block_groups)  # [B, m] group indices
    block_owner = owner[block_groups[:, 0]]
    nb = block_groups.shape[0]
    calls = -(-nb // BLOCKS)
    sel = np.resize(np.arange(nb), calls * BLOCKS) if nb % BLOCKS else np.arange(nb)
    sel = sel.reshape(calls, BLOCKS)
    # A [calls, m, K]: token t, block b of call c = group block_groups[sel[c, b], t]
    gidx = block_groups[sel]  # [calls, 64, m]
    a_bits = groups[gidx].transpose(0, 2, 1, 3).reshape(calls, m, K_ID)
    a_all = to_gpu(_bf16(a_bits))
    # identity weight: code 0x38 (1.0) on the diagonal; per-call block scales
    w_q = torch.zeros((K_ID, K_ID), dtype=torch.uint8, device=a_all.device)
    w_q.diagonal().fill_(0x38)
    scale_pow = exps[block_owner[sel]]  # [calls, 64]
    w_s_all = np.ones((calls, BLOCKS, BLOCKS), dtype=np.float32)
    w_s_all[:, np.arange(BLOCKS), np.arange(BLOCKS)] = np.ldexp(np.float32(1.0), scale_pow).astype(np.float32)
    w_s_all = to_gpu(w_s_all)
    c_all = torch.empty((calls, m, K_ID), dtype=torch.bfloat16, device=a_all.device)
    for c in range(calls):
        fp8bq.gemm_fused(a_all[c], w_q, w_s_all[c], out=c_all[c])
    torch.cuda.synchronize()
    got = c_all.to(torch.float64).cpu().numpy()  # [calls, m, K]
    # expected from the oracle's codes and scales: bf16(fp32(dec * s * 2^e)),
    # the exact product rounded once to fp32 (the kernel's fma) and once to bf16
    dec = e4m3_decode(oq[gidx])  # [calls, 64, m, 128]
    sc = os_[gidx].astype(np.float64) * np.ldexp(1.0, scale_pow)[:, :, None]
    exact = dec * sc[..., None]
    want = bf16_rne(exact.astype(np.float32).astype(np.float64))
    want = want.transpose(0, 2, 1, 3).reshape(calls, m, K_ID)
    bad = np.argwhere(got != want)
    if bad.size:
        c, t, n = bad[0]
        b, j = divmod(int(n), 128)
        g = gidx[c, b, t]
        raise AssertionError(
            f"M={m}: {bad.shape[0]} outputs differ; first: call {c} token {t} column {n}: max pattern "
            f"{groups[g, 0]:#06x}, x pattern {groups[g, j]:#06x}, gpu {got[c, t, n]!r}, want {want[c, t, n]!r}")
