"""CPU oracle for W8A8 block-FP8 activation quantisation and GEMM.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
HIP path is checked against. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it; the
product path (``memory_bound_w8a8_amd``) never does, and the two share no code.

What it computes, and where the pages state it:

* The method is the "W8A8 Block FP8" linear layer whose five (N, K) weight
  shapes are listed in page 2 (ownding.com L20 report), section 8 "L20 FP8
  Kernel tuning experiment"; page 1 (SmartX blog), section "single-stream
  optimisation", says the W8A8 backend quantises activations on every call
  (the W8A16 Marlin backend is faster at one stream because it skips that
  step). The pages name the scheme but never define its numerics; the
  numerics used here are the DeepSeek-style block-FP8 scheme that page 2's
  tuning script defaults to: OCP e4m3fn codes, weight scale per 128x128 block,
  activation scale per token per 128-wide K group, scale = amax / 448 in fp32,
  bf16 output.

Modules:

* ``e4m3``  -- OCP OFP8 e4m3fn decode (closed form) and round-to-nearest-even
  encode (nearest-value search, ties to the even code).
* ``quant`` -- per-token 1x128 activation quantisation and per-128x128-block
  weight quantisation, fp32 arithmetic exactly as numpy float32 (IEEE RN).
* ``gemm``  -- the dequantised block-scaled product in fp64, whole or at
  sampled output positions.
* ``w8a16`` -- the weight-only variant (bf16 activation x block-FP8 weight,
  page 1's W8A16 backend), fp64, whole or sampled.
* ``scoring`` -- two-stage vocabulary scoring: exact top-k of coarse logits
  and exact fp64 rescoring of the survivors (page 1's FP8-screen,
  BF16-score scheme).

Every function is pinned by ``-m "not gpu"`` tests against something other
than itself (torch's float8_e4m3fn casts, exact rational brute force, closed
forms and invariants). No function here is "parity unpinned".
"""

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode_rne, e4m3_values
from .quant import quant_act_ref, quant_weight_ref
from .gemm import gemm_ref, gemm_ref_at
from .w8a16 import gemm_w8a16_ref, gemm_w8a16_ref_at
from .scoring import bf16_key, rescore_ref, topk_ref

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode_rne",
    "e4m3_values",
    "quant_act_ref",
    "quant_weight_ref",
    "gemm_ref",
    "gemm_ref_at",
    "gemm_w8a16_ref",
    "gemm_w8a16_ref_at",
    "bf16_key",
    "topk_ref",
    "rescore_ref",
]
