/*
 * fp8bq -- W8A8 block-FP8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The operation is the weight GEMM of a dense decoder's linear layer,
 * y = x W^T, with W stored as "W8A8 Block FP8" of shape (N, K) -- page 2
 * (ownding.com, "Qwen3.8-27B-FP8 + MTP tuning report on two NVIDIA L20"),
 * section 8 "L20 FP8 Kernel tuning experiment", which lists the five logged
 * (N, K) shapes; page 1 (SmartX blog, "Qwen3.8-27B performance
 * optimisation"), section "single-stream optimisation", which says the W8A8
 * backend quantises the activation on every call; and the same page's
 * section "operator optimisation", which puts about 89% of each decode step
 * in these weight-reading matmuls.
 *
 * Number format (the pages say only "FP8"; the block scheme is the
 * DeepSeek-style one page 2's tuning script targets):
 *   - codes are OCP e4m3fn bytes (bias 7, max 448, no infinities, 0x7F/0xFF
 *     NaN); a value is decode(code) * scale;
 *   - activations: one fp32 scale per token per 128 consecutive K entries;
 *   - weights: one fp32 scale per 128 x 128 block (rows 128b.., cols 128g..);
 *   - scale = amax / 448 (IEEE fp32 division), 1.0 for an all-zero group;
 *     codes = RNE(clamp(x / scale, -448, 448)).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers on the current HIP device; all
 *     tensors are dense row-major. The caller owns every buffer; the library
 *     allocates nothing, keeps no pointer after return and has no state
 *     beyond a per-device capability check and the static scratch array of
 *     fp8bq_topk_bf16_noalloc (with its per-device address).
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work
 *     on it and return without synchronising; faults during execution
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued. On
 *     error nothing is launched and a negative fp8bq_status is returned.
 *   - M == 0 or N == 0 is a quick return (FP8BQ_OK, nothing launched).
 *   - Outputs must not alias inputs. NaN/Inf activations or weights and
 *     NaN weight codes (0x7F, 0xFF) give unspecified results.
 *   - Calls on different streams are independent and may run concurrently.
 */
#ifndef FP8BQ_H
#define FP8BQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8bq_status {
    FP8BQ_OK = 0,
    FP8BQ_ERR_NULL = -1,   /* a required pointer is NULL                     */
    FP8BQ_ERR_SHAPE = -2,  /* a size is negative, K % 128 != 0, or too large  */
    FP8BQ_ERR_ALIGN = -3,  /* code/bf16 pointer not 16-B aligned, fp32 not 4-B */
    FP8BQ_ERR_DEVICE = -4, /* no HIP device, or the current device is not gfx950 */
    FP8BQ_ERR_LAUNCH = -5, /* the HIP runtime rejected a kernel launch        */
    FP8BQ_ERR_SCRATCH = -6 /* the request needs more than the library's static
                              scratch buffer (fp8bq_topk_bf16_noalloc)       */
} fp8bq_status;

/*
 * Per-token activation quantisation (page 1, "single-stream optimisation":
 * the per-call activation-quantisation launch of the W8A8 backend).
 *
 *   A_bf16   [M, K] bf16, read.
 *   A_fp8    [M, K] uint8 e4m3fn codes, written.
 *   A_scales [M, K/128] fp32, written; A_scales[m, g] is the scale of
 *            A_bf16[m, 128g .. 128g+127].
 * Bit-exact: codes and scales equal the definition above for every finite
 * input (fp32 amax, IEEE division, RNE to e4m3fn, signed zero kept).
 * Errors: NULL pointer; M < 0, K < 0 or K % 128 != 0; M*K > 2^40; A_bf16 or
 * A_fp8 not 16-B aligned, A_scales not 4-B aligned; device not gfx950.
 */
int fp8bq_quant_act(int64_t M, int64_t K, const void *A_bf16, void *A_fp8, float *A_scales,
                    void *stream);

/*
 * Per-128x128-block weight quantisation (page 2, section 8: the weights of
 * each logged shape are stored as W8A8 block FP8). The pages' checkpoints
 * arrive pre-quantised; this call builds such weights from fp32 on the GPU.
 *
 *   W_f32    [N, K] fp32, read. N arbitrary: the last row block may be short.
 *   W_fp8    [N, K] uint8 e4m3fn codes, written.
 *   W_scales [ceil(N/128), K/128] fp32, written.
 * Bit-exact with the same rule as fp8bq_quant_act, amax taken per block.
 * Errors: as fp8bq_quant_act (W_f32 must be 16-B aligned).
 */
int fp8bq_quant_weight(int64_t N, int64_t K, const float *W_f32, void *W_fp8, float *W_scales,
                       void *stream);

/*
 * Block-scaled FP8 GEMM (page 2, section 8: the W8A8 block-FP8 matmul of
 * shape (N, K) at batch size M; page 1, "operator optimisation": the
 * weight-reading matmuls that bound the decode step).
 *
 *   C[m, n] = sum_g A_scales[m, g] * W_scales[n / 128, g]
 *                   * sum_{k = 128g}^{128g+127} dec(A_fp8[m, k]) * dec(W_fp8[n, k])
 *
 *   A_fp8    [M, K] uint8 codes,  A_scales [M, K/128] fp32          (read)
 *   W_fp8    [N, K] uint8 codes,  W_scales [ceil(N/128), K/128] fp32 (read)
 *   C_bf16   [M, N] bf16, written, fp32 accumulation rounded to bf16 RNE.
 * Every M >= 1 is served by a kernel chosen from explicit ranges (no
 * nearest-size table): M <= 64 streams the weights once, and so does
 * 65 <= M <= 80 where one round of 256 workgroups covers N with at most 32
 * weight rows each and K <= 5120 (five 16-token sub-tiles; the registers
 * of larger shapes spill); every other M > 64 runs the
 * LDS-tiled MFMA kernel, whose tile shape (64x64 up to 256x256 tokens x
 * weight rows) follows from (M, N) by the number of rounds of workgroups
 * its grid needs on the 256 CUs (for the 192x256 and 256x256 tiles a last
 * round of at most 128 tiles runs as a second launch of column halves,
 * with the same per-output summation order). The summation order differs
 * from the fp64
 * definition; results agree within fp32 accumulation plus bf16 rounding.
 * Two identical calls give bitwise-identical C (no atomics).
 * K == 0 writes zeros. Errors: NULL pointer; negative size; K % 128 != 0;
 * M*K, N*K or M*N > 2^40; M > 64 with K >= 2^24 (the tiled kernel's limit);
 * code/bf16 pointers not 16-B aligned, scale pointers not 4-B aligned;
 * device not gfx950.
 */
int fp8bq_gemm(int64_t M, int64_t N, int64_t K, const void *A_fp8, const float *A_scales,
               const void *W_fp8, const float *W_scales, void *C_bf16, void *stream);

/*
 * Kernel-path introspection for tests and profiling. Returns the path
 * fp8bq_gemm would take for (M, N, K) -- FP8BQ_PATH_STREAM for the
 * weight-streaming split-K kernels, FP8BQ_PATH_TILED for the LDS-tiled MFMA
 * kernel -- or a negative status for invalid sizes.
 */
enum { FP8BQ_PATH_NONE = 0, FP8BQ_PATH_STREAM = 1, FP8BQ_PATH_TILED = 2 };
/* Tile shapes of the tiled kernel (tokens x weight rows), accepted by
 * fp8bq_gemm_forced only; FP8BQ_PATH_TILED picks one from (M, N). */
enum {
  FP8BQ_PATH_TILED_128x128 = 3,
  FP8BQ_PATH_TILED_128x256 = 4,
  FP8BQ_PATH_TILED_192x256 = 5,
  FP8BQ_PATH_TILED_256x256 = 6,
  FP8BQ_PATH_TILED_64x128 = 7,
  FP8BQ_PATH_TILED_128x64 = 8,
  FP8BQ_PATH_TILED_64x64 = 9
};
int fp8bq_gemm_path(int64_t M, int64_t N, int64_t K);

/*
 * The tile shape the LDS-tiled kernel takes for (M, N, K), as the
 * FP8BQ_PATH_TILED_* value fp8bq_gemm_forced accepts (fp8bq_gemm uses it
 * where it does not stream; any M >= 1 is answered): the shape with the least grid
 * rounds on the 256 CUs times measured step cost. FP8BQ_PATH_NONE for
 * M == 0 or N == 0, a negative status for invalid sizes. Host-only: no
 * device is needed.
 */
int fp8bq_gemm_tile_shape(int64_t M, int64_t N, int64_t K);

/*
 * fp8bq_gemm with the kernel path forced (FP8BQ_PATH_STREAM requires
 * M <= 128, as one launch where fp8bq_gemm streams and otherwise two
 * launches past 64 tokens; FP8BQ_PATH_TILED and the
 * FP8BQ_PATH_TILED_* shapes accept any M). For cross-checking the paths and
 * tile shapes at the same M: every tile shape sums each output in the same
 * order, so their results are bitwise equal. Same arguments, semantics and errors as fp8bq_gemm, plus
 * FP8BQ_ERR_SHAPE for a path that cannot serve M.
 */
int fp8bq_gemm_forced(int path, int64_t M, int64_t N, int64_t K, const void *A_fp8,
                      const float *A_scales, const void *W_fp8, const float *W_scales,
                      void *C_bf16, void *stream);

/*
 * fp8bq_gemm with a caller-provided device workspace: the same operation,
 * arguments, semantics and errors, plus the workspace. Where fp8bq_gemm
 * runs the LDS-tiled kernel (beyond 64 tokens) and its tiles would leave
 * CUs idle (M = 65..~256 on the logged shapes: 20..136 tiles for 256 CUs),
 * the workspace lets the K/128 groups of each tile be split over several
 * workgroups: each part writes an fp32 partial tile into the workspace and
 * a second launch adds the parts in a fixed order and rounds to bf16 (RNE).
 * Identical calls give identical bits; the split changes the summation
 * order, so results can differ from fp8bq_gemm's in the last bits (both
 * agree with the fp64 definition within fp32 accumulation plus bf16
 * rounding).
 *   workspace        device memory, 16-B aligned, workspace_bytes long (NULL
 *                    only with workspace_bytes == 0), not overlapping the
 *                    other arguments; overwritten. Calls sharing a
 *                    workspace must be ordered (same stream).
 *   workspace_bytes  >= fp8bq_gemm_workspace_bytes(M, N, K) > 0: the split
 *                    plan runs; otherwise exactly fp8bq_gemm's kernels run
 *                    (bitwise equal to fp8bq_gemm).
 * Errors: as fp8bq_gemm, plus FP8BQ_ERR_SHAPE for workspace_bytes < 0,
 * FP8BQ_ERR_NULL for a NULL workspace with workspace_bytes > 0 and
 * FP8BQ_ERR_ALIGN for a workspace not 16-B aligned.
 *
 * fp8bq_gemm_workspace_bytes: the bytes the split plan for (M, N, K) takes
 * (split x M x N x 4), 0 where fp8bq_gemm_ws does not split, or a negative
 * status for invalid sizes. Host-only: no device is needed.
 *
 * fp8bq_gemm_ws_forced: the split plan with the tile shape (an
 * FP8BQ_PATH_TILED_* value: 128x128, 128x256, 64x128, 128x64 or 64x64)
 * and the number of K parts (2 .. min(64, K/128)) forced, workspace_bytes
 * >= split x M x N x 4; split == 1 runs fp8bq_gemm_forced(path, ...). For
 * cross-checking plans: FP8BQ_ERR_SHAPE for a shape or split it cannot
 * run, or a grid of tiles x split workgroups of 2^31 or more.
 */
int64_t fp8bq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int fp8bq_gemm_ws(int64_t M, int64_t N, int64_t K, const void *A_fp8, const float *A_scales,
                  const void *W_fp8, const float *W_scales, void *C_bf16, void *workspace,
                  int64_t workspace_bytes, void *stream);
int fp8bq_gemm_ws_forced(int path, int split, int64_t M, int64_t N, int64_t K, const void *A_fp8,
                         const float *A_scales, const void *W_fp8, const float *W_scales,
                         void *C_bf16, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Activation quantisation and block-FP8 GEMM in one launch (page 1, SmartX
 * blog, "single-stream optimisation": the W8A8 backend's per-call
 * activation quantisation is a separate launch at every linear layer; here
 * it runs inside the GEMM).
 *
 *   C = fp8bq_gemm(fp8bq_quant_act(A_bf16), W_fp8, W_scales)
 *
 *   A_bf16   [M, K] bf16, read; 1 <= M <= 8
 *   W_fp8, W_scales as fp8bq_gemm; C_bf16 [M, N] bf16, written.
 * Up to 8 tokens: every workgroup of the launch quantises the whole
 * activation, which beyond 8 tokens no longer hides under the weight stream
 * of the narrower weights (two launches are faster there).
 * The codes and scales formed inside are exactly those fp8bq_quant_act
 * writes, and C is bitwise the two-call result; they are not stored.
 * M == 0 or N == 0 is a quick return; K == 0 writes zeros. Errors: NULL
 * pointer; negative size; K % 128 != 0; M > 8; K > 9216 (more than 72
 * groups); M*K, N*K or M*N > 2^40; A_bf16, W_fp8 or C_bf16 not 16-B aligned,
 * W_scales not 4-B aligned; device not gfx950.
 */
int fp8bq_gemm_fused(int64_t M, int64_t N, int64_t K, const void *A_bf16, const void *W_fp8,
                     const float *W_scales, void *C_bf16, void *stream);

/*
 * Weight-only block-FP8 GEMM (page 1, SmartX blog, "single-stream
 * optimisation": the W8A16 backend keeps the activation in 16 bits and skips
 * the per-call activation quantisation; it was the faster backend at one
 * stream and the slower one at high concurrency, so this entry point serves
 * small batches only).
 *
 *   C[m, n] = sum_g W_scales[n / 128, g]
 *                   * sum_{k = 128g}^{128g+127} A[m, k] * dec(W_fp8[n, k])
 *
 *   A_bf16   [M, K] bf16, read; 1 <= M <= 16
 *   W_fp8    [N, K] uint8 codes, W_scales [ceil(N/128), K/128] fp32 (read),
 *            the same weights fp8bq_gemm takes
 *   C_bf16   [M, N] bf16, written; products exact, fp32 accumulation,
 *            rounded to bf16 RNE. Two identical calls give identical bits.
 * M == 0 or N == 0 is a quick return; K == 0 writes zeros. Errors: NULL
 * pointer; negative size; K % 128 != 0; M > 16; K > 9216 (more than 72
 * groups); M*K, N*K or M*N > 2^40; A_bf16, W_fp8 or C_bf16 not 16-B aligned,
 * W_scales not 4-B aligned; device not gfx950.
 */
int fp8bq_gemm_w8a16(int64_t M, int64_t N, int64_t K, const void *A_bf16, const void *W_fp8,
                     const float *W_scales, void *C_bf16, void *stream);

/*
 * Two-stage vocabulary scoring (page 1, SmartX blog, "single-stream
 * optimisation": the draft head reads the whole vocabulary projection every
 * step; all candidates are screened with FP8 scores and only the survivors
 * are scored exactly in BF16). Stage 1 is fp8bq_gemm / fp8bq_gemm_fused of
 * the hidden state with the FP8 vocabulary projection, giving coarse bf16
 * logits [M, V]; stage 2 is fp8bq_topk_bf16; stage 3 is fp8bq_rescore_bf16
 * against the BF16 projection.
 *
 * Order (the pages give none): bf16 values compare by their bit pattern
 * mapped to a monotone unsigned key (negative patterns inverted, positive
 * ones with the top bit set; so -0 ranks just below +0, and NaN patterns
 * rank by their bits like any other), equal keys by the lower index.
 */

/*
 * Bytes of device workspace fp8bq_topk_bf16 needs for (M, V, k), or a
 * negative status for sizes it rejects. The size depends on M, V and k only.
 */
int64_t fp8bq_topk_workspace_bytes(int64_t M, int64_t V, int64_t k);

/*
 * Exact top-k of each row of bf16 logits.
 *
 *   logits_bf16  [M, V] bf16, read.
 *   workspace    device scratch of at least workspace_bytes >=
 *                fp8bq_topk_workspace_bytes(M, V, k) bytes; contents on
 *                entry are ignored, on return unspecified. Calls that share
 *                a workspace must be ordered (same stream).
 *   idx_out      [M, k] int32, written: the k best entries of each row in
 *                order (best first), by the order above.
 *   val_bf16_out [M, k] bf16, written: their logit bit patterns.
 * Bit-exact (an order, no arithmetic); deterministic.
 * M == 0 is a quick return. Errors: k < 1, k > 256 or k > V; V >= 2^31;
 * M*V > 2^40; more than 2^21 first-level workgroups (M * ceil(ceil(V / 1024)
 * / G), G = min(4, floor(1024 / k))); workspace_bytes too small; NULL
 * pointer; logits, workspace or
 * val_bf16_out not 16-B aligned, idx_out not 4-B aligned; device not gfx950.
 */
int fp8bq_topk_bf16(int64_t M, int64_t V, int64_t k, const void *logits_bf16, void *workspace,
                    int64_t workspace_bytes, int32_t *idx_out, void *val_bf16_out, void *stream);

/*
 * fp8bq_topk_bf16 for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that must not call hipMalloc, harnesses
 * that forbid allocation. It takes no workspace; its kernels use a static
 * device array of the library instead, FP8BQ_TOPK_SCRATCH_BYTES (4 MiB) on
 * each GPU it runs on, held until the process ends. Its address is looked
 * up once per device on the first call there; the call allocates nothing.
 *
 *   logits_bf16, idx_out, val_bf16_out, k, M, V: as fp8bq_topk_bf16, with
 *   identical results (bitwise).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or host threads without ordering) race and
 * must be ordered by the caller. The array's contents need no clearing (the
 * kernels ignore them on entry) and are unspecified after a call.
 * Errors: as fp8bq_topk_bf16 (no workspace arguments), plus
 * FP8BQ_ERR_SCRATCH when fp8bq_topk_workspace_bytes(M, V, k) exceeds
 * FP8BQ_TOPK_SCRATCH_BYTES (e.g. V = 152064, k = 64 serves M <= 199).
 */
#define FP8BQ_TOPK_SCRATCH_BYTES (4 << 20)
int fp8bq_topk_bf16_noalloc(int64_t M, int64_t V, int64_t k, const void *logits_bf16, int32_t *idx_out,
                            void *val_bf16_out, void *stream);

/*
 * Exact scores of the survivors and each row's pick.
 *
 *   h_bf16     [M, K] bf16 hidden states, read.
 *   W_bf16     [V, K] bf16 vocabulary projection, read (rows idx only).
 *   idx        [M, k] int32 survivor indices, read (e.g. fp8bq_topk_bf16's).
 *   scores_out [M, k] fp32, written: scores_out[m, j] =
 *              sum_k h[m, k] * W[idx[m, j], k], products exact in fp32, fp32
 *              accumulation in a fixed order (bitwise repeatable); NaN for an
 *              index outside [0, V), whose row is not read.
 *   pick_out   [M] int32, written: the index of the survivor with the largest
 *              score (ties to the lower index); NaN scores are never picked;
 *              -1 when all of a row's scores are NaN.
 * M == 0 is a quick return; K == 0 scores 0. Errors: k < 1; K % 8 != 0;
 * V >= 2^31; M*K, V*K or M*k > 2^40; more than 2^21 rows or survivor groups
 * of 16; NULL pointer (h_bf16 and W_bf16 may be NULL when K == 0); h_bf16 or
 * W_bf16 not 16-B aligned, idx, scores_out or pick_out not 4-B aligned;
 * device not gfx950.
 */
int fp8bq_rescore_bf16(int64_t M, int64_t K, int64_t V, int64_t k, const void *h_bf16,
                       const void *W_bf16, const int32_t *idx, float *scores_out,
                       int32_t *pick_out, void *stream);

/*
 * Measurement kernels: what this machine delivers, to read the GEMM's
 * roofline fractions against besides the published peaks (page 1, SmartX
 * blog: "single-stream optimisation" reports bytes per decode step over time
 * against a calibrated bandwidth; "test background" calibrates the tools
 * first). All five only read their inputs and write `sink`.
 *
 * fp8bq_mb_read: streaming read of `bytes` bytes at `buf` (bytes % 16 == 0,
 *   buf 16-B aligned) by `grid` (1..65536) workgroups of 512 threads,
 *   consecutive lanes on consecutive 16-byte units, non-temporal loads,
 *   twelve in flight per lane. sink [grid] uint32 (out): the XOR of the
 *   32-bit words each workgroup read; XORed together they equal the XOR of
 *   every word of the buffer. bytes == 0 (buf may then be NULL) writes
 *   zeros.
 * fp8bq_mb_empty: one launch of an empty kernel, `grid` (1..2^20)
 *   workgroups of `block` (64..1024, a multiple of 64) threads.
 * fp8bq_mb_mfma_e4m3: `grid` (1..65536) workgroups of 4 waves, each wave
 *   8 independent chains of `iters` (0..2^24) V_MFMA_F32_16X16X128_F8F6F4
 *   (2 * 16 * 16 * 128 flop each) with every operand byte the e4m3 code
 *   `code` (0..255, not a NaN code). sink [grid * 256] fp32 (out): thread t
 *   writes 4096 * iters * decode(code)^2 (exact while that fits in fp32's
 *   24 bits).
 * fp8bq_mb_mfma_e4m3_data: the same loop with operands read from `codes`
 *   (device, 16-B aligned, 32768 bytes of e4m3 codes, no NaN code; NaN codes
 *   give unspecified sums): in every wave, chain u's first and second operand
 *   in lane l are the 32 bytes at codes + 32 * ((2u + o) * 64 + l), o = 0, 1.
 *   Output element i of lane l (row 4 (l / 16) + i, column l % 16) is
 *   sum over q = 0..3, b = 0..31 of decode(first[16q + row][b]) *
 *   decode(second[16q + column][b]) (lane L's bytes first[L][.], second[L][.]),
 *   accumulated `iters` times in fp32; thread t writes the sum of its 32
 *   elements (8 chains x 4) to sink[t] (sink [grid * 256] fp32). With
 *   quantised Gaussian codes this is the matrix-core rate a GEMM's data
 *   allows (its switching activity sets the clock the chip can hold).
 * fp8bq_mb_mfma_e4m3_scaled: the block-scaled GEMM's inner loop on the same
 *   operands (page 2, ownding.com L20 report, section 8: the W8A8 block FP8
 *   GEMM, one scale per 128-wide group): every MFMA starts from zero and its
 *   4 results per lane are folded into the chain's running sums by 4 fp32
 *   FMAs with `scale`, one MFMA later, so that the matrix core and the VALU
 *   share each SIMD as in fp8bq_gemm's tiled kernel. sink: `scale` times
 *   the sums of fp8bq_mb_mfma_e4m3_data (exact when both are). The rate
 *   this loop reaches is the most a GEMM that scales every group's products
 *   in fp32 can get from the matrix cores.
 * Errors as for the GEMM: FP8BQ_ERR_SHAPE, _NULL, _ALIGN, _DEVICE, _LAUNCH.
 */
int fp8bq_mb_read(const void *buf, int64_t bytes, int grid, unsigned *sink, void *stream);
int fp8bq_mb_empty(int grid, int block, void *stream);
int fp8bq_mb_mfma_e4m3(int grid, int iters, int code, float *sink, void *stream);
int fp8bq_mb_mfma_e4m3_data(int grid, int iters, const void *codes, float *sink, void *stream);
int fp8bq_mb_mfma_e4m3_scaled(int grid, int iters, const void *codes, float scale, float *sink,
                              void *stream);

/* Human-readable name of a status code; never NULL. */
const char *fp8bq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_H */
