"""The top-k entry point that allocates nothing (fp8bq_topk_bf16_noalloc),
through the C ABI: bitwise the same indices and values as fp8bq_topk_bf16
with a caller workspace, on consecutive calls that share the library's
static scratch array (the second smaller than the first, so stale contents
of the first are present), at the largest size the scratch serves, and
against the oracle's top-k."""

import numpy as np
import pytest
import torch

import memory_bound_w8a8_amd as fp8bq
import workloads
from oracle import topk_ref
from helpers import to_gpu

pytestmark = pytest.mark.gpu


def _logits(m, v, kind, seed):
    bits = workloads.logit_bits(m, v, kind, seed)
    return to_gpu(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)), bits


def _both(logits, k):
    m = logits.shape[0]
    idx_w, val_w = fp8bq.topk(logits, k)
    idx_n = torch.full((m, k), -7, dtype=torch.int32, device=logits.device)
    val_n = torch.zeros((m, k), dtype=torch.bfloat16, device=logits.device)
    fp8bq.topk_noalloc(logits, k, idx_n, val_n)
    torch.cuda.synchronize()
    return idx_w, val_w, idx_n, val_n


@pytest.mark.parametrize("calls", [[(16, workloads.VOCAB, 64, "normal", 1), (3, 5000, 17, "bits", 2)],
                                   [(4, 70000, 256, "ties", 3), (1, 1024, 1, "normal", 4)]])
def test_noalloc_matches_workspace_entry_on_consecutive_calls(calls):
    for m, v, k, kind, seed in calls:
        logits, bits = _logits(m, v, kind, seed)
        idx_w, val_w, idx_n, val_n = _both(logits, k)
        assert torch.equal(idx_n, idx_w), f"indices differ: M={m} V={v} k={k}"
        assert torch.equal(val_n.view(torch.int16), val_w.view(torch.int16)), f"values differ: M={m} V={v} k={k}"
        want_idx, _ = topk_ref(bits, k)
        assert np.array_equal(idx_n.cpu().numpy(), want_idx), f"oracle: M={m} V={v} k={k}"


def test_noalloc_largest_size_the_scratch_serves():
    v, k = workloads.VOCAB, 64
    per_row = fp8bq.topk_workspace_bytes(1, v, k)
    m = fp8bq.TOPK_SCRATCH_BYTES // per_row  # 199 rows
    logits, _ = _logits(m, v, "normal", 5)
    idx_w, val_w, idx_n, val_n = _both(logits, k)
    assert torch.equal(idx_n, idx_w) and torch.equal(val_n.view(torch.int16), val_w.view(torch.int16))
    with pytest.raises(fp8bq.Fp8bqError):
        big, _ = _logits(m + 1, v, "normal", 6)
        fp8bq.topk_noalloc(big, k, torch.empty((m + 1, k), dtype=torch.int32, device=big.device),
                           torch.empty((m + 1, k), dtype=torch.bfloat16, device=big.device))
