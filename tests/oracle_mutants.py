"""Planted mistakes in the oracle, for checking that its pins can fail.

    python tests/oracle_mutants.py <name>

patches one plausible mistake into the oracle's modules (in this process
only), then runs the oracle pin file that covers the patched function with
pytest -x and exits with pytest's status: 1 means a pin caught the mistake.
tests/test_mutants_oracle.py runs every mutant and requires that status.
The oracle's files are never modified.
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path[:0] = [ROOT, HERE]

import oracle  # noqa: E402
import oracle.e4m3 as e4m3  # noqa: E402
import oracle.gemm as gemm  # noqa: E402
import oracle.quant as quant  # noqa: E402
import oracle.scoring as scoring  # noqa: E402
import oracle.w8a16 as w8a16  # noqa: E402

F32 = np.float32


def _set(name, fn, *modules):
    """Rebind `name` in the oracle package and in each module that uses it."""
    setattr(oracle, name, fn)
    for mod in modules:
        setattr(mod, name, fn)


def _encode_variant(tie_up=False, keep_sign=True):
    good = e4m3.e4m3_encode_rne

    def enc(v):
        v = np.asarray(v, dtype=F32)
        if not tie_up and keep_sign:
            return good(v)
        mag = np.abs(v).astype(np.float64)
        lower = np.searchsorted(e4m3._POS_VALUES, mag, side="right") - 1
        has_upper = lower < 0x7E
        mid = e4m3._MIDPOINTS[np.minimum(lower, 0x7D)]
        if tie_up:  # ties away from zero
            up = has_upper & (mag >= mid)
        else:
            up = has_upper & ((mag > mid) | ((mag == mid) & ((lower & 1) == 1)))
        code = np.where(up, lower + 1, lower).astype(np.uint8)
        sign = (np.signbit(v) & (mag > 0) if not keep_sign else np.signbit(v)).astype(np.uint8) << 7
        return (code | sign).astype(np.uint8)

    return enc


def _table_variant(sub_exp=-6, bias=7):
    t = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
            continue
        mag = (m / 8) * 2.0 ** sub_exp if e == 0 else (1 + m / 8) * 2.0 ** (e - bias)
        t[c] = -mag if s else mag
    return t


def _gemm_variant(ws_index="block", sa_shift=0, drop_last=False, ws_transposed=False):
    def ref(a_q, a_s, w_q, w_s):
        a_q, a_s, w_q, w_s, m, n, k, g = gemm._check(a_q, a_s, w_q, w_s)
        a_dec = e4m3.e4m3_decode(a_q)
        w_dec = e4m3.e4m3_decode(w_q)
        wsf = w_s.astype(np.float64)
        if ws_transposed and wsf.shape[0] == wsf.shape[1]:
            wsf = wsf.T
        if ws_index == "block":
            sw_rows = np.repeat(wsf, 128, axis=0)[:n]
        else:  # row n uses scale row n % blocks
            sw_rows = wsf[np.arange(n) % wsf.shape[0]]
        c = np.zeros((m, n))
        for gi in range(g - (1 if drop_last and g > 1 else 0)):
            ks = slice(gi * 128, gi * 128 + 128)
            scale = a_s[:, (gi + sa_shift) % g].astype(np.float64)[:, None] * sw_rows[None, :, gi]
            c += scale * (a_dec[:, ks] @ w_dec[:, ks].T)
        return c

    def ref_at(a_q, a_s, w_q, w_s, rows, cols):
        return ref(a_q, a_s, w_q, w_s)[np.asarray(rows), np.asarray(cols)]

    return ref, ref_at


def _quant_scale_eps(amax):
    amax = amax.astype(F32)
    s = np.divide(amax, F32(448), dtype=F32)
    return np.where(amax > 0, s, F32(2.0 ** -20)).astype(F32)


def _quant_act_signed_max(a):
    x = quant._as_float32(a)
    m, k = x.shape
    grp = x.reshape(m, k // 128, 128)
    amax = np.abs(np.max(grp, axis=2))  # max, not max-abs
    s = quant._scale_from_amax(amax)
    return quant._encode_scaled(grp, s[:, :, None]).reshape(m, k), s


def _quant_weight_rowwise(w):
    x = quant._as_float32(w)
    n, k = x.shape
    codes, scales = quant.quant_act_ref(x)  # per row instead of per block
    nb = -(-n // 128)
    return codes, scales[::128][:nb]


def _topk_ties_high(bits, k):
    bits = np.asarray(bits, dtype=np.uint16)
    m, v = bits.shape
    key = scoring.bf16_key(bits)
    idx = np.empty((m, k), dtype=np.int64)
    for i in range(m):
        order = np.lexsort((-np.arange(v), -key[i].astype(np.int64)))
        idx[i] = order[:k]
    return idx, np.take_along_axis(bits, idx, axis=1)


def _rescore_ties_high(h, w, idx):
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    scores = np.einsum("mk,mjk->mj", h, w[idx])
    pick = np.array([idx[i, max(range(idx.shape[1]), key=lambda j: (scores[i, j], idx[i, j]))]
                     for i in range(idx.shape[0])])
    return scores, pick


def _w8a16_no_scale(a, w_q, w_s):
    a = np.asarray(a, dtype=np.float64)
    return a @ e4m3.e4m3_decode(w_q).T


def apply(name):
    if name == "quant_multiplies_by_reciprocal":
        quant._encode_scaled = lambda x, s: e4m3.e4m3_encode_rne(
            np.clip(np.multiply(x, np.divide(F32(1), s, dtype=F32), dtype=F32), F32(-448), F32(448)))
    elif name == "quant_zero_group_scale_eps":
        quant._scale_from_amax = _quant_scale_eps
    elif name == "quant_signed_max":
        _set("quant_act_ref", _quant_act_signed_max, quant)
    elif name == "quant_weight_per_row":
        _set("quant_weight_ref", _quant_weight_rowwise, quant)
    elif name == "encode_ties_away":
        enc = _encode_variant(tie_up=True)
        _set("e4m3_encode_rne", enc, e4m3, quant)
    elif name == "encode_drops_negative_zero":
        enc = _encode_variant(keep_sign=False)
        _set("e4m3_encode_rne", enc, e4m3, quant)
    elif name == "decode_subnormal_exponent":
        e4m3._TABLE = _table_variant(sub_exp=-7)
    elif name == "decode_exponent_bias":
        e4m3._TABLE = _table_variant(bias=8)
    elif name == "gemm_weight_scale_transposed":
        ref, ref_at = _gemm_variant(ws_transposed=True)
        _set("gemm_ref", ref, gemm)
        _set("gemm_ref_at", ref_at, gemm)
    elif name == "gemm_weight_scale_row_modulo":
        ref, ref_at = _gemm_variant(ws_index="modulo")
        _set("gemm_ref", ref, gemm)
        _set("gemm_ref_at", ref_at, gemm)
    elif name == "gemm_activation_scale_next_group":
        ref, ref_at = _gemm_variant(sa_shift=1)
        _set("gemm_ref", ref, gemm)
        _set("gemm_ref_at", ref_at, gemm)
    elif name == "gemm_drops_last_group":
        ref, ref_at = _gemm_variant(drop_last=True)
        _set("gemm_ref", ref, gemm)
        _set("gemm_ref_at", ref_at, gemm)
    elif name == "topk_ties_to_higher_index":
        _set("topk_ref", _topk_ties_high, scoring)
    elif name == "rescore_pick_ties_to_higher_index":
        _set("rescore_ref", _rescore_ties_high, scoring)
    elif name == "w8a16_drops_weight_scale":
        _set("gemm_w8a16_ref", _w8a16_no_scale, w8a16)
    else:
        raise SystemExit(f"unknown mutant {name}")


# mutant -> the pin file expected to catch it (the driver runs that file)
MUTANTS = {
    "quant_multiplies_by_reciprocal": "test_oracle_quant.py",
    "quant_zero_group_scale_eps": "test_oracle_quant.py",
    "quant_signed_max": "test_oracle_quant.py",
    "quant_weight_per_row": "test_oracle_quant.py",
    "encode_ties_away": "test_oracle_e4m3.py",
    "encode_drops_negative_zero": "test_oracle_e4m3.py",
    "decode_subnormal_exponent": "test_oracle_e4m3.py",
    "decode_exponent_bias": "test_oracle_e4m3.py",
    "gemm_weight_scale_transposed": "test_oracle_gemm.py",
    "gemm_weight_scale_row_modulo": "test_oracle_gemm.py",
    "gemm_activation_scale_next_group": "test_oracle_gemm.py",
    "gemm_drops_last_group": "test_oracle_gemm.py",
    "topk_ties_to_higher_index": "test_oracle_scoring.py",
    "rescore_pick_ties_to_higher_index": "test_oracle_scoring.py",
    "w8a16_drops_weight_scale": "test_oracle_w8a16.py",
}


if __name__ == "__main__":
    import pytest

    name = sys.argv[1]
    apply(name)
    sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "--no-header", os.path.join(HERE, MUTANTS[name])]))
