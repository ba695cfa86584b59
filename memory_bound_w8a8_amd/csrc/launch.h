// Host-side launchers of the fp8bq kernels (internal to libfp8bq.so).
// Arguments are validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

hipError_t launch_quant_act(int64_t m, int64_t k, const void* a, void* aq, float* as, hipStream_t stream);
hipError_t launch_quant_weight(int64_t n, int64_t k, const float* w, void* wq, float* ws, hipStream_t stream);

// Weight-streaming split-K kernel, 1 <= m <= 64, and 65 <= m <= 80 where
// stream_wide_serves(m, n, k) (hipErrorInvalidValue otherwise).
hipError_t launch_gemm_stream(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                              const void* wq, const float* ws, void* c, hipStream_t stream);

// LDS-tiled MFMA kernel, any m >= 1. shape -1 picks the tile shape from
// (m, n) (tiled_shape); 0..6 force 128x128, 128x256, 192x256, 256x256,
// 64x128, 128x64, 64x64. tiled_shape also returns the chosen shape's cost
// of one K step (1/100 us) through step_cost when that is not null.
int tiled_shape(int64_t m, int64_t n, int64_t* step_cost);

// K-split tiled path (fp8bq_gemm_ws): shape as above (one of the
// gemm_tiled_kernel shapes 0, 1, 4, 5, 6) and split > 1 parts of the K
// groups per tile, or shape = tiled_shape(m, n) and split = 1 (no split);
// cost in 1/100 us. launch_gemm_split needs part = split x m x n fp32
// (16-byte aligned) and runs the partial tiles, then their fixed-order sum.
struct SplitPlan {
  int shape = 0;
  int split = 1;
  int64_t cost = 0;
};
SplitPlan split_plan(int64_t m, int64_t n, int64_t k);
// Tiles of tile shape `shape` (0..6, as for launch_gemm_tiled) over M x N.
int64_t tile_grid(int64_t m, int64_t n, int shape);
hipError_t launch_gemm_split(int64_t m, int64_t n, int64_t k, const void* aq, const float* as, const void* wq,
                             const float* ws, void* c, float* part, int shape, int split, hipStream_t stream);
hipError_t launch_gemm_tiled(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                             const void* wq, const float* ws, void* c, hipStream_t stream, int shape = -1);

// The small-M entry points below serve 1 <= m <= 16 and K/128 groups within
// the streaming instance table.
bool small_m_supported(int64_t m, int64_t n, int64_t k);
// Whether 65..96 tokens on (N, K) have a streaming instance (at most two
// 16-row tiles per workgroup).
bool stream_wide_serves(int64_t m, int64_t n, int64_t k);
// Whether 33..64 tokens on (N, K) stream with long per-wave K ranges (8..9
// groups) over 2 row tiles, where fp8bq_gemm_ws splits K instead.
bool stream_deep_k(int64_t m, int64_t n, int64_t k);

// Activation quantisation fused into the streaming GEMM (bf16 activation in).
hipError_t launch_gemm_fused(int64_t m, int64_t n, int64_t k, const void* a, const void* wq, const float* ws, void* c,
                             hipStream_t stream);

// Weight-only (bf16 activation) streaming kernel.
hipError_t launch_gemm_w8a16(int64_t m, int64_t n, int64_t k, const void* a, const void* wq, const float* ws, void* c,
                             hipStream_t stream);

// Two-stage vocabulary scoring (scoring.hip). topk: 1 <= k <= 256, k <= v;
// the workspace holds topk_workspace_bytes(m, v, k) bytes; the grids hold
// topk_grid_blocks / rescore_grid_blocks workgroups of 1024 threads.
int64_t topk_workspace_bytes(int64_t m, int64_t v, int64_t k);
int64_t topk_grid_blocks(int64_t m, int64_t v, int64_t k);
int64_t rescore_grid_blocks(int64_t m, int64_t k);
hipError_t launch_topk(int64_t m, int64_t v, int k, const void* logits, void* workspace, int* idx, void* val,
                       hipStream_t stream);
// fp8bq_topk_bf16_noalloc: the same kernels with the library's static
// per-GPU scratch array (kTopkScratchBytes) as their workspace. The caller
// checks topk_workspace_bytes(m, v, k) <= kTopkScratchBytes first.
constexpr int64_t kTopkScratchBytes = int64_t(4) << 20;
hipError_t topk_scratch_address(void** out);
hipError_t launch_topk_noalloc(int64_t m, int64_t v, int k, const void* logits, int* idx, void* val,
                               hipStream_t stream);
hipError_t launch_rescore(int64_t m, int64_t kdim, int64_t v, int64_t k, const void* h, const void* w,
                          const int* idx, float* scores, int* pick, hipStream_t stream);

// Kernel-choice log (FP8BQ_LOG=1): prints each distinct (entry, M, N, K)
// -> kernel description once to stderr; a no-op otherwise.
void dispatch_log(const char* entry, int64_t m, int64_t n, int64_t k, const char* kernel);

// Measurement kernels (microbench.hip): streaming read of `bytes` (a
// multiple of 16) with `grid` workgroups of 512 threads, one XOR word per
// workgroup into sink[grid]; an empty kernel; `grid` workgroups of 4 waves
// each running 8 x iters FP8 MFMAs on the e4m3 code `code`, one float per
// thread into sink[grid * 256].
hipError_t launch_mb_read(const void* buf, int64_t bytes, int grid, unsigned* sink, hipStream_t stream);
hipError_t launch_mb_empty(int grid, int block, hipStream_t stream);
hipError_t launch_mb_mfma(int grid, int iters, unsigned code, float* sink, hipStream_t stream);
hipError_t launch_mb_mfma_data(int grid, int iters, const void* codes, float* sink, hipStream_t stream);
hipError_t launch_mb_mfma_scaled(int grid, int iters, const void* codes, float scale, float* sink,
                                 hipStream_t stream);

// C = 0 (used for K == 0).
hipError_t launch_fill_zero_bf16(int64_t count, void* c, hipStream_t stream);

}  // namespace fp8bq
