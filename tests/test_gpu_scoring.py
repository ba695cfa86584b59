"""GPU parity of two-stage vocabulary scoring (fp8bq_topk_bf16,
fp8bq_rescore_bf16, and the fused GEMM in front of them) against the oracle's
topk_ref / rescore_ref / gemm_ref, through the C ABI.

Top-k is an order, so it must match bit for bit: indices and values. Scores
are fp32 dot products of bf16 rows; their bound against the fp64 oracle is
derived from the kernel's summation order (see _score_bound). Inputs come
from the seeded generators in `workloads`."""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
from helpers import BF16_U, RMS_TOL, assert_gemm_close, bf16_to_f64, to_gpu
from oracle import gemm_ref, gemm_ref_at, quant_act_ref, quant_weight_ref, rescore_ref, topk_ref
import workloads

pytestmark = pytest.mark.gpu


def _bits_to_bf16_gpu(bits: np.ndarray) -> torch.Tensor:
    return to_gpu(bits.view(np.int16)).view(torch.bfloat16)


def _gpu_topk(bits: np.ndarray, k: int):
    idx, val = fp8bq.topk(_bits_to_bf16_gpu(bits), k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.view(torch.int16).cpu().numpy().view(np.uint16)


def _check_topk(bits: np.ndarray, k: int, what: str):
    idx, val = _gpu_topk(bits, k)
    ref_idx, ref_val = topk_ref(bits, k)
    assert np.array_equal(idx.astype(np.int64), ref_idx), what
    assert np.array_equal(val, ref_val), what


@pytest.mark.parametrize("kind", ["normal", "ties", "bits"])
@pytest.mark.parametrize("m,v,k", [(1, 1000, 1), (3, 4096, 5), (2, 4097, 64), (5, 9000, 50), (1, 8, 8),
                                   (2, 300, 256), (4, 20000, 255), (1, 65536 + 3, 129), (2, 30000, 17)])
def test_topk_bit_exact(kind, m, v, k):
    bits = workloads.logit_bits(m, v, kind, seed=7)
    _check_topk(bits, k, f"{kind} M={m} V={v} k={k}")


@pytest.mark.parametrize("k,v", [(1, 4096 * 2048 + 11), (2, 4096 * 2048 + 11), (64, 4096 * 64 * 2 + 3),
                                 (256, 3 * 4096 * 16 + 5)])
def test_topk_multi_level_merge(k, v):
    # a merge workgroup takes 4096 / p lists (p = power of two >= k): k = 1
    # fills one to capacity (2049 lists); the others need two merge levels
    bits = workloads.logit_bits(1, v, "normal", seed=k)
    _check_topk(bits, k, f"V={v} k={k}")


def test_topk_all_equal_and_signed_zero():
    # every entry equal: the lowest indices win, in order
    bits = np.full((2, 5000), 0x3F80, dtype=np.uint16)
    bits[1, :] = 0x8000  # -0 everywhere ...
    bits[1, 4321] = 0x0000  # ... except one +0, which ranks above -0
    idx, val = _gpu_topk(bits, 10)
    assert np.array_equal(idx[0], np.arange(10))
    assert idx[1, 0] == 4321 and np.array_equal(idx[1, 1:], np.arange(9))
    assert np.array_equal(val[1, 1:], np.full(9, 0x8000, dtype=np.uint16))
    _check_topk(bits, 10, "constant rows")


def test_topk_full_size_and_deterministic():
    m, v, k = 16, workloads.VOCAB, workloads.SURVIVORS
    bits = workloads.logit_bits(m, v, "normal", seed=1)
    idx1, val1 = _gpu_topk(bits, k)
    idx2, val2 = _gpu_topk(bits, k)
    assert np.array_equal(idx1, idx2) and np.array_equal(val1, val2)
    ref_idx, ref_val = topk_ref(bits, k)
    assert np.array_equal(idx1.astype(np.int64), ref_idx)
    assert np.array_equal(val1, ref_val)


def test_topk_caller_workspace_reused():
    m, v, k = 4, 50000, 32
    ws = torch.empty(fp8bq.topk_workspace_bytes(m, v, k), dtype=torch.uint8, device="cuda")
    for seed in (1, 2):
        bits = workloads.logit_bits(m, v, "bits", seed=seed)
        idx, val = fp8bq.topk(_bits_to_bf16_gpu(bits), k, workspace=ws)
        torch.cuda.synchronize()
        ref_idx, _ = topk_ref(bits, k)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), ref_idx)


def _score_bound(h: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """|fp32 score - exact| bound: each lane sums 8 * ceil(K / 512) exact
    products in one fp32 chain, then 6 butterfly additions; every rounding
    is at most 2^-24 relative to a partial sum bounded by sum |h w|, so
    (chain + 6) * 2^-24 * sum |h w| (x 1.01 for second-order terms)."""
    kdim = h.shape[1]
    chain = 8 * -(-kdim // 512) + 6
    mag = np.einsum("mk,mjk->mj", np.abs(h), np.abs(w_rows))
    return 1.01 * chain * 2.0 ** -24 * mag + 1e-30


def _rescore_case(m, kdim, v, k, seed):
    h = workloads.activation(m, v, kdim)
    w = workloads.to_bf16(workloads.weight(v, kdim))
    idx = workloads.survivor_indices(m, v, k, seed)
    return h, w, idx


def _run_rescore(h, w, idx):
    scores, pick = fp8bq.rescore(to_gpu(h), to_gpu(w), to_gpu(idx))
    torch.cuda.synchronize()
    return scores.cpu().numpy(), pick.cpu().numpy()


def _check_rescore(h, w, idx, scores, pick, what):
    h64 = h.float().numpy().astype(np.float64)
    rows, inv = np.unique(idx.astype(np.int64), return_inverse=True)
    w_rows = w[torch.from_numpy(rows)].float().numpy().astype(np.float64)
    inv = inv.reshape(idx.shape)
    ref, ref_pick = rescore_ref(h64, w_rows, inv)
    bound = _score_bound(h64, w_rows[inv])
    err = np.abs(scores.astype(np.float64) - ref)
    assert np.all(err <= bound), f"{what}: worst excess {np.max(err - bound)!r}"
    # the pick is the best survivor by the GPU's own scores (ties to the
    # lower index) ...
    for r in range(idx.shape[0]):
        best = max(range(idx.shape[1]), key=lambda j: (scores[r, j], -int(idx[r, j])))
        assert pick[r] == idx[r, best], (what, r)
    # ... and within the score bound of the exact best
    j_pick = np.array([list(idx[r]).index(pick[r]) for r in range(idx.shape[0])])
    best_ref = ref.max(axis=1)
    got_ref = ref[np.arange(idx.shape[0]), j_pick]
    assert np.all(got_ref >= best_ref - 2 * bound.max(axis=1)), what
    # a clear exact winner is the oracle's pick
    second = np.sort(ref, axis=1)[:, -2] if ref.shape[1] > 1 else np.full(ref.shape[0], -np.inf)
    clear = best_ref - second > 2 * bound.max(axis=1)
    assert np.array_equal(pick[clear].astype(np.int64), rows[ref_pick[clear]]), what


@pytest.mark.parametrize("m,kdim,v,k", [(1, 5120, 2000, 64), (3, 1024, 700, 1), (16, 2048, 5000, 17),
                                        (2, 8, 100, 16), (5, 4096 + 8, 3000, 100), (1, 128, 64, 64)])
def test_rescore_parity(m, kdim, v, k):
    h, w, idx = _rescore_case(m, kdim, v, k, seed=3)
    scores, pick = _run_rescore(h, w, idx)
    _check_rescore(h, w, idx, scores, pick, f"M={m} K={kdim} V={v} k={k}")


def test_rescore_full_size_and_deterministic():
    m, kdim, v, k = 16, workloads.HIDDEN, workloads.VOCAB, workloads.SURVIVORS
    h, w, idx = _rescore_case(m, kdim, v, k, seed=5)
    s1, p1 = _run_rescore(h, w, idx)
    s2, p2 = _run_rescore(h, w, idx)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32)) and np.array_equal(p1, p2)
    _check_rescore(h, w, idx, s1, p1, "full size")


def test_rescore_ties_invalid_indices_and_k_zero():
    m, kdim, v = 2, 256, 50
    h = workloads.activation(m, v, kdim)
    w = workloads.to_bf16(workloads.weight(v, kdim))
    # rows 30 and 10 equal, aligned with h[0]: the clear, tied best of row 0
    w[30] = workloads.to_bf16(0.5 * np.sign(h[0].float().numpy()))
    w[10] = w[30]
    idx = np.array([[30, 10, 3, -1], [v, -5, v + 100, 7]], dtype=np.int32)
    scores, pick = _run_rescore(h, w, idx)
    assert scores[0, 0] == scores[0, 1] and scores[0, 0] > scores[0, 2]
    assert np.isnan(scores[0, 3]) and np.isnan(scores[1, :3]).all() and not np.isnan(scores[1, 3])
    assert pick[0] == 10  # equal best scores: the lower index
    assert pick[1] == 7
    # a row whose survivors are all out of range picks -1
    scores, pick = _run_rescore(h[:1], w, np.array([[v, -1]], dtype=np.int32))
    assert np.isnan(scores).all() and pick[0] == -1
    # K == 0: every score is 0, the lowest index wins
    z = torch.empty((1, 0), dtype=torch.bfloat16)
    scores, pick = _run_rescore(z, torch.empty((v, 0), dtype=torch.bfloat16), np.array([[9, 4, 12]], dtype=np.int32))
    assert np.array_equal(scores, np.zeros((1, 3), np.float32)) and pick[0] == 4


def _gemm_tol(ref: np.ndarray) -> np.ndarray:
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return RMS_TOL * rms + BF16_U * np.abs(ref)


@pytest.mark.parametrize("m,v,kdim,k", [(1, 20000, 1024, 64), (5, 9000 + 77, 2048, 50), (16, 4096, 512, 8),
                                        (24, 3000, 1024, 16)])
def test_two_stage_pipeline(m, v, kdim, k):
    # oracle: coarse logits = block-FP8 GEMM of the quantised hidden state and
    # the FP8 projection; exact scores = bf16 hidden state x bf16 projection
    h = workloads.activation(m, v, kdim)
    w32 = workloads.weight(v, kdim)
    w_bf = workloads.to_bf16(w32)
    w_q, w_s = quant_weight_ref(w32)
    a_q, a_s = quant_act_ref(h.float().numpy())
    coarse = gemm_ref(a_q, a_s, w_q, w_s)
    exact = h.float().numpy().astype(np.float64) @ w_bf.float().numpy().astype(np.float64).T

    pick, idx, scores = fp8bq.two_stage(to_gpu(h), to_gpu(w_q), to_gpu(w_s), to_gpu(w_bf), k)
    torch.cuda.synchronize()
    pick, idx, scores = pick.cpu().numpy(), idx.cpu().numpy().astype(np.int64), scores.cpu().numpy()

    tol = _gemm_tol(coarse)
    for r in range(m):
        sel = np.zeros(v, dtype=bool)
        sel[idx[r]] = True
        assert sel.sum() == k, "survivors must be distinct"
        # a valid top-k of the coarse logits, up to their tolerance
        assert np.min(coarse[r, sel] + tol[r, sel]) >= np.max(coarse[r, ~sel] - tol[r, ~sel])
        # scores: the exact products, within the fp32 bound
        w_rows = w_bf[torch.from_numpy(idx[r])].float().numpy().astype(np.float64)[None]
        bound = _score_bound(h[r : r + 1].float().numpy().astype(np.float64), w_rows)[0]
        assert np.all(np.abs(scores[r] - exact[r, idx[r]]) <= bound)
        # the pick: a survivor whose exact score is within the bound of the best survivor's
        assert pick[r] in idx[r]
        assert exact[r, pick[r]] >= exact[r, idx[r]].max() - 2 * bound.max()


def test_coarse_logits_vocabulary_size_sampled():
    # stage 1 at the full vocabulary size (V = 152064 rows: the row-range
    # kernel runs several rounds of workgroups), fused quantisation + GEMM,
    # against the oracle on sampled weight row blocks and all tokens
    v, kdim = workloads.VOCAB, workloads.HIDDEN
    w_q, w_s = fp8bq.quant_weight(to_gpu(workloads.weight(v, kdim)))
    nb = (v + 127) // 128
    rng = np.random.default_rng(11)
    blocks = sorted({0, nb - 1, *rng.integers(0, nb, size=4).tolist()})
    ow = [quant_weight_ref(workloads.weight_block(v, kdim, b)) for b in blocks]
    wq_cat = np.concatenate([oq for oq, _ in ow])
    ws_cat = np.concatenate([os_ for _, os_ in ow])
    cols_local = np.concatenate([128 * i + np.arange(oq.shape[0]) for i, (oq, _) in enumerate(ow)])
    cols_global = np.concatenate([128 * b + np.arange(oq.shape[0]) for b, (oq, _) in zip(blocks, ow)])
    for m in (1, 4, 8):
        h = workloads.activation(m, v, kdim)
        logits = fp8bq.gemm_fused(to_gpu(h), w_q, w_s)
        torch.cuda.synchronize()
        a_q, a_s = quant_act_ref(h.float().numpy())
        rr, cc = np.meshgrid(np.arange(m), np.arange(len(cols_local)), indexing="ij")
        ref = gemm_ref_at(a_q, a_s, wq_cat, ws_cat, rr.ravel(), cols_local[cc.ravel()])
        got = bf16_to_f64(logits[:, torch.from_numpy(cols_global).to(logits.device)]).ravel()
        assert_gemm_close(got, ref, what=f"coarse logits M={m} V={v}")
