// C ABI of libfp8bq: host-side validation and kernel dispatch. The contract
// of every entry point is documented in include/fp8bq.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "fp8bq.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;  // bound on M*K, N*K, M*N
constexpr int64_t kStreamMaxM = 64;              // streaming kernels: 1..64 tokens per launch on any shape
constexpr int64_t kStreamSplitMaxM = 128;        // forced streaming path up to 128 tokens (two launches past 64
                                                 // where the 65..80 instances do not serve)
constexpr int64_t kTiledMaxK = int64_t(1) << 24; // tiled kernel: 32-bit offsets within a 256-row tile
constexpr int kMaxDevices = 64;
constexpr int64_t kSmallMaxM = 16;               // weight-only path: one 16-token tile
constexpr int64_t kFusedMaxM = 8;                // fused path: quantisation layouts for up to 8 tokens
constexpr int64_t kSmallMaxK = 72 * 128;         // groups within their instance tables
constexpr int64_t kTopkMaxK = 256;               // survivors per row
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;  // vocabulary indices are int32
constexpr int64_t kMaxGridBlocks = int64_t(1) << 21;   // 1024-thread workgroups in one 1-D grid

// Per-device capability cache: 0 = unknown, 1 = gfx950, -1 = not usable.
std::atomic<int> g_device_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8BQ_ERR_DEVICE;
  if (dev >= kMaxDevices) return FP8BQ_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    state = -1;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      state = 1;
    g_device_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8BQ_OK : FP8BQ_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool product_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxElems / a; }

int launch_status(hipError_t e) { return e == hipSuccess ? FP8BQ_OK : FP8BQ_ERR_LAUNCH; }

int check_gemm_args(int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales, const void* W_fp8,
                    const float* W_scales, void* C_bf16) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_OK;
  if (C_bf16 == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(C_bf16, 16)) return FP8BQ_ERR_ALIGN;
  if (K == 0) return FP8BQ_OK;
  if (A_fp8 == nullptr || A_scales == nullptr || W_fp8 == nullptr || W_scales == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(A_fp8, 16) || !aligned(W_fp8, 16) || !aligned(A_scales, 4) || !aligned(W_scales, 4))
    return FP8BQ_ERR_ALIGN;
  return FP8BQ_OK;
}

// 1..64 tokens stream the weights once, and 65..80 too where the five
// sub-tile instances fit in registers (at most 2 row tiles per workgroup
// and 5 groups per wave: N <= 8192 and K <= 5120; 7-12% faster there than
// the tiled kernel). Beyond, the tiled kernel, whose 4-wave 64 x 64 to
// 128 x 128 tiles keep the CUs filled at 65..128 tokens (streaming the
// weights twice, tokens 0..63 and then the rest, measured 15-30% slower on
// the N = 5120..8192 shapes and 15% on N = 17408).
int gemm_path(int64_t M, int64_t N, int64_t K) {
  if (M <= kStreamMaxM || fp8bq::stream_wide_serves(M, N, K)) return FP8BQ_PATH_STREAM;
  return FP8BQ_PATH_TILED;
}

hipError_t launch_stream_split(int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales,
                               const void* W_fp8, const float* W_scales, void* C_bf16, hipStream_t s) {
  if (M <= kStreamMaxM || fp8bq::stream_wide_serves(M, N, K))
    return fp8bq::launch_gemm_stream(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, s);
  const hipError_t e = fp8bq::launch_gemm_stream(kStreamMaxM, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, s);
  if (e != hipSuccess) return e;
  return fp8bq::launch_gemm_stream(M - kStreamMaxM, N, K, static_cast<const unsigned char*>(A_fp8) + kStreamMaxM * K,
                                   A_scales + kStreamMaxM * (K / 128), W_fp8, W_scales,
                                   static_cast<unsigned short*>(C_bf16) + kStreamMaxM * N, s);
}

int run_gemm(int path, int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales,
             const void* W_fp8, const float* W_scales, void* C_bf16, void* stream) {
  int st = check_gemm_args(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16);
  if (st != FP8BQ_OK) return st;
  const bool tiled = path == FP8BQ_PATH_TILED || (path >= FP8BQ_PATH_TILED_128x128 && path <= FP8BQ_PATH_TILED_64x64);
  if (path == FP8BQ_PATH_STREAM && M > kStreamSplitMaxM) return FP8BQ_ERR_SHAPE;
  if (tiled && K >= kTiledMaxK) return FP8BQ_ERR_SHAPE;
  if (path != FP8BQ_PATH_STREAM && !tiled) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_OK;
  st = check_device();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return launch_status(fp8bq::launch_fill_zero_bf16(M * N, C_bf16, s));
  if (path == FP8BQ_PATH_STREAM)
    return launch_status(launch_stream_split(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, s));
  const int shape = path == FP8BQ_PATH_TILED ? -1 : path - FP8BQ_PATH_TILED_128x128;
  return launch_status(fp8bq::launch_gemm_tiled(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, s, shape));
}

// Workspace bytes the K-split plan of fp8bq_gemm_ws needs for a valid
// (M, N, K) with M, N, K > 0 (0 when the plan does not split).
// Beyond the streaming kernels' reach the plan competes with the unsplit
// tiled plan; at 33..64 tokens it replaces streaming only where that is
// bound by long per-wave K ranges (stream_deep_k).
int64_t split_workspace_bytes(int64_t M, int64_t N, int64_t K, fp8bq::SplitPlan* plan) {
  if (K >= kTiledMaxK) return 0;
  if (gemm_path(M, N, K) != FP8BQ_PATH_TILED && !fp8bq::stream_deep_k(M, N, K)) return 0;
  *plan = fp8bq::split_plan(M, N, K);
  return plan->split > 1 ? plan->split * M * N * 4 : 0;
}

int check_workspace(const void* workspace, int64_t workspace_bytes) {
  if (workspace_bytes < 0) return FP8BQ_ERR_SHAPE;
  if (workspace_bytes > 0 && workspace == nullptr) return FP8BQ_ERR_NULL;
  if (workspace != nullptr && !aligned(workspace, 16)) return FP8BQ_ERR_ALIGN;
  return FP8BQ_OK;
}

}  // namespace

extern "C" {

int fp8bq_quant_act(int64_t M, int64_t K, const void* A_bf16, void* A_fp8, float* A_scales, void* stream) {
  if (M < 0 || K < 0 || K % 128 != 0 || !product_ok(M, K)) return FP8BQ_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8BQ_OK;
  if (A_bf16 == nullptr || A_fp8 == nullptr || A_scales == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(A_bf16, 16) || !aligned(A_fp8, 16) || !aligned(A_scales, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_quant_act(M, K, A_bf16, A_fp8, A_scales, static_cast<hipStream_t>(stream)));
}

int fp8bq_quant_weight(int64_t N, int64_t K, const float* W_f32, void* W_fp8, float* W_scales, void* stream) {
  if (N < 0 || K < 0 || K % 128 != 0 || !product_ok(N, K)) return FP8BQ_ERR_SHAPE;
  if ((N + 127) / 128 > 65535) return FP8BQ_ERR_SHAPE;  // row blocks form the grid's y dimension
  if (N == 0 || K == 0) return FP8BQ_OK;
  if (W_f32 == nullptr || W_fp8 == nullptr || W_scales == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(W_f32, 16) || !aligned(W_fp8, 16) || !aligned(W_scales, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_quant_weight(N, K, W_f32, W_fp8, W_scales, static_cast<hipStream_t>(stream)));
}

int fp8bq_gemm(int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales, const void* W_fp8,
               const float* W_scales, void* C_bf16, void* stream) {
  if (M < 0 || N < 0) return FP8BQ_ERR_SHAPE;
  return run_gemm(gemm_path(M, N, K), M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, stream);
}

int fp8bq_gemm_forced(int path, int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales,
                      const void* W_fp8, const float* W_scales, void* C_bf16, void* stream) {
  return run_gemm(path, M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, stream);
}

int64_t fp8bq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0) return 0;
  fp8bq::SplitPlan plan;
  return split_workspace_bytes(M, N, K, &plan);
}

int fp8bq_gemm_ws(int64_t M, int64_t N, int64_t K, const void* A_fp8, const float* A_scales, const void* W_fp8,
                  const float* W_scales, void* C_bf16, void* workspace, int64_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return FP8BQ_ERR_SHAPE;
  int st = check_gemm_args(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16);
  if (st != FP8BQ_OK) return st;
  st = check_workspace(workspace, workspace_bytes);
  if (st != FP8BQ_OK) return st;
  if (M > 0 && N > 0 && K > 0) {
    fp8bq::SplitPlan plan;
    const int64_t need = split_workspace_bytes(M, N, K, &plan);
    if (need > 0 && workspace_bytes >= need) {
      st = check_device();
      if (st != FP8BQ_OK) return st;
      return launch_status(fp8bq::launch_gemm_split(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16,
                                                    static_cast<float*>(workspace), plan.shape, plan.split,
                                                    static_cast<hipStream_t>(stream)));
    }
  }
  return run_gemm(gemm_path(M, N, K), M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, stream);
}

int fp8bq_gemm_ws_forced(int path, int split, int64_t M, int64_t N, int64_t K, const void* A_fp8,
                         const float* A_scales, const void* W_fp8, const float* W_scales, void* C_bf16,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (split == 1) {
    const int st = check_workspace(workspace, workspace_bytes);
    if (st != FP8BQ_OK) return st;
    return run_gemm(path, M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16, stream);
  }
  if (M < 0 || N < 0) return FP8BQ_ERR_SHAPE;
  int st = check_gemm_args(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16);
  if (st != FP8BQ_OK) return st;
  st = check_workspace(workspace, workspace_bytes);
  if (st != FP8BQ_OK) return st;
  const int shape = path - FP8BQ_PATH_TILED_128x128;
  const bool splits = shape == 0 || shape == 1 || shape == 4 || shape == 5 || shape == 6;
  if (!splits || split < 2 || split > 64 || split > K / 128 || K >= kTiledMaxK) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_OK;
  // the grid, tiles x split workgroups, must stay within 2^31
  if (fp8bq::tile_grid(M, N, shape) * split >= (int64_t(1) << 31)) return FP8BQ_ERR_SHAPE;
  if (workspace_bytes < split * M * N * 4) return FP8BQ_ERR_SHAPE;
  st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_gemm_split(M, N, K, A_fp8, A_scales, W_fp8, W_scales, C_bf16,
                                                static_cast<float*>(workspace), shape, split,
                                                static_cast<hipStream_t>(stream)));
}

int fp8bq_gemm_path(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_PATH_NONE;
  return gemm_path(M, N, K);
}

int fp8bq_gemm_tile_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_PATH_NONE;
  return FP8BQ_PATH_TILED_128x128 + fp8bq::tiled_shape(M, N, nullptr);
}

int fp8bq_gemm_fused(int64_t M, int64_t N, int64_t K, const void* A_bf16, const void* W_fp8, const float* W_scales,
                     void* C_bf16, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M > kFusedMaxM || K > kSmallMaxK) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_OK;
  if (C_bf16 == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(C_bf16, 16)) return FP8BQ_ERR_ALIGN;
  if (K > 0) {
    if (A_bf16 == nullptr || W_fp8 == nullptr || W_scales == nullptr) return FP8BQ_ERR_NULL;
    if (!aligned(A_bf16, 16) || !aligned(W_fp8, 16) || !aligned(W_scales, 4)) return FP8BQ_ERR_ALIGN;
  }
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return launch_status(fp8bq::launch_fill_zero_bf16(M * N, C_bf16, s));
  if (!fp8bq::small_m_supported(M, N, K)) return FP8BQ_ERR_SHAPE;
  return launch_status(fp8bq::launch_gemm_fused(M, N, K, A_bf16, W_fp8, W_scales, C_bf16, s));
}

int fp8bq_gemm_w8a16(int64_t M, int64_t N, int64_t K, const void* A_bf16, const void* W_fp8, const float* W_scales,
                     void* C_bf16, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N)) return FP8BQ_ERR_SHAPE;
  if (M > kSmallMaxM || K > kSmallMaxK) return FP8BQ_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BQ_OK;
  if (C_bf16 == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(C_bf16, 16)) return FP8BQ_ERR_ALIGN;
  if (K > 0) {
    if (A_bf16 == nullptr || W_fp8 == nullptr || W_scales == nullptr) return FP8BQ_ERR_NULL;
    if (!aligned(A_bf16, 16) || !aligned(W_fp8, 16) || !aligned(W_scales, 4)) return FP8BQ_ERR_ALIGN;
  }
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return launch_status(fp8bq::launch_fill_zero_bf16(M * N, C_bf16, s));
  if (!fp8bq::small_m_supported(M, N, K)) return FP8BQ_ERR_SHAPE;
  return launch_status(fp8bq::launch_gemm_w8a16(M, N, K, A_bf16, W_fp8, W_scales, C_bf16, s));
}

int64_t fp8bq_topk_workspace_bytes(int64_t M, int64_t V, int64_t k) {
  if (M < 0 || V < 0 || V > kMaxIndex || k < 1 || k > kTopkMaxK || k > V || !product_ok(M, V)) return FP8BQ_ERR_SHAPE;
  return fp8bq::topk_workspace_bytes(M, V, k);
}

int fp8bq_topk_bf16(int64_t M, int64_t V, int64_t k, const void* logits_bf16, void* workspace,
                    int64_t workspace_bytes, int32_t* idx_out, void* val_bf16_out, void* stream) {
  if (M < 0 || V < 0 || V > kMaxIndex || k < 1 || k > kTopkMaxK || k > V || !product_ok(M, V)) return FP8BQ_ERR_SHAPE;
  if (fp8bq::topk_grid_blocks(M, V, k) > kMaxGridBlocks) return FP8BQ_ERR_SHAPE;
  if (M == 0) return FP8BQ_OK;
  if (workspace_bytes < fp8bq::topk_workspace_bytes(M, V, k)) return FP8BQ_ERR_SHAPE;
  if (logits_bf16 == nullptr || workspace == nullptr || idx_out == nullptr || val_bf16_out == nullptr)
    return FP8BQ_ERR_NULL;
  if (!aligned(logits_bf16, 16) || !aligned(workspace, 16) || !aligned(idx_out, 4) || !aligned(val_bf16_out, 16))
    return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_topk(M, V, static_cast<int>(k), logits_bf16, workspace, idx_out, val_bf16_out,
                                          static_cast<hipStream_t>(stream)));
}

int fp8bq_topk_bf16_noalloc(int64_t M, int64_t V, int64_t k, const void* logits_bf16, int32_t* idx_out,
                            void* val_bf16_out, void* stream) {
  if (M < 0 || V < 0 || V > kMaxIndex || k < 1 || k > kTopkMaxK || k > V || !product_ok(M, V)) return FP8BQ_ERR_SHAPE;
  if (fp8bq::topk_grid_blocks(M, V, k) > kMaxGridBlocks) return FP8BQ_ERR_SHAPE;
  if (M == 0) return FP8BQ_OK;
  if (fp8bq::topk_workspace_bytes(M, V, k) > fp8bq::kTopkScratchBytes) return FP8BQ_ERR_SCRATCH;
  if (logits_bf16 == nullptr || idx_out == nullptr || val_bf16_out == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(logits_bf16, 16) || !aligned(idx_out, 4) || !aligned(val_bf16_out, 16)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_topk_noalloc(M, V, static_cast<int>(k), logits_bf16, idx_out, val_bf16_out,
                                                  static_cast<hipStream_t>(stream)));
}

int fp8bq_rescore_bf16(int64_t M, int64_t K, int64_t V, int64_t k, const void* h_bf16, const void* W_bf16,
                       const int32_t* idx, float* scores_out, int32_t* pick_out, void* stream) {
  if (M < 0 || K < 0 || K % 8 != 0 || V < 0 || V > kMaxIndex || k < 1) return FP8BQ_ERR_SHAPE;
  if (!product_ok(M, K) || !product_ok(V, K) || !product_ok(M, k)) return FP8BQ_ERR_SHAPE;
  if (fp8bq::rescore_grid_blocks(M, k) > kMaxGridBlocks || M > kMaxGridBlocks) return FP8BQ_ERR_SHAPE;
  if (M == 0) return FP8BQ_OK;
  if (idx == nullptr || scores_out == nullptr || pick_out == nullptr) return FP8BQ_ERR_NULL;
  if (K > 0 && (h_bf16 == nullptr || W_bf16 == nullptr)) return FP8BQ_ERR_NULL;
  if (!aligned(idx, 4) || !aligned(scores_out, 4) || !aligned(pick_out, 4)) return FP8BQ_ERR_ALIGN;
  if (K > 0 && (!aligned(h_bf16, 16) || !aligned(W_bf16, 16))) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_rescore(M, K, V, k, h_bf16, W_bf16, idx, scores_out, pick_out,
                                             static_cast<hipStream_t>(stream)));
}

const char* fp8bq_status_string(int status) {
  switch (status) {
    case FP8BQ_OK: return "ok";
    case FP8BQ_ERR_NULL: return "null pointer argument";
    case FP8BQ_ERR_SHAPE: return "invalid size (negative, K % 128 != 0, too large, or path cannot serve M)";
    case FP8BQ_ERR_ALIGN: return "misaligned pointer (codes/bf16 need 16 B, fp32 scales 4 B)";
    case FP8BQ_ERR_DEVICE: return "no usable HIP device (gfx950 required)";
    case FP8BQ_ERR_LAUNCH: return "kernel launch failed";
    case FP8BQ_ERR_SCRATCH: return "request needs more than the library's static scratch buffer (4 MiB per GPU)";
    default: return "unknown status";
  }
}

int fp8bq_mb_read(const void* buf, int64_t bytes, int grid, unsigned* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || grid < 1 || grid > 65536) return FP8BQ_ERR_SHAPE;
  if ((buf == nullptr && bytes != 0) || sink == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_mb_read(buf, bytes, grid, sink, static_cast<hipStream_t>(stream)));
}

int fp8bq_mb_empty(int grid, int block, void* stream) {
  if (grid < 1 || grid > (1 << 20) || block < 64 || block > 1024 || block % 64 != 0) return FP8BQ_ERR_SHAPE;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_mb_empty(grid, block, static_cast<hipStream_t>(stream)));
}

int fp8bq_mb_mfma_e4m3(int grid, int iters, int code, float* sink, void* stream) {
  if (grid < 1 || grid > 65536 || iters < 0 || iters > (1 << 24) || code < 0 || code > 255 ||
      (code & 0x7f) == 0x7f)
    return FP8BQ_ERR_SHAPE;
  if (sink == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(sink, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(
      fp8bq::launch_mb_mfma(grid, iters, static_cast<unsigned>(code), sink, static_cast<hipStream_t>(stream)));
}

int fp8bq_mb_mfma_e4m3_data(int grid, int iters, const void* codes, float* sink, void* stream) {
  if (grid < 1 || grid > 65536 || iters < 0 || iters > (1 << 24)) return FP8BQ_ERR_SHAPE;
  if (codes == nullptr || sink == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(sink, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(fp8bq::launch_mb_mfma_data(grid, iters, codes, sink, static_cast<hipStream_t>(stream)));
}

int fp8bq_mb_mfma_e4m3_scaled(int grid, int iters, const void* codes, float scale, float* sink, void* stream) {
  if (grid < 1 || grid > 65536 || iters < 0 || iters > (1 << 24)) return FP8BQ_ERR_SHAPE;
  if (codes == nullptr || sink == nullptr) return FP8BQ_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(sink, 4)) return FP8BQ_ERR_ALIGN;
  const int st = check_device();
  if (st != FP8BQ_OK) return st;
  return launch_status(
      fp8bq::launch_mb_mfma_scaled(grid, iters, codes, scale, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
