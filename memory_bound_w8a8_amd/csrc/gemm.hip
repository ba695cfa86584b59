// Kernel instances and launch configuration of the block-FP8 GEMM.
#include "device_common.h"
#include "gemm_stream.h"
#include "gemm_tiled.h"
#include "launch.h"

namespace fp8bq {

namespace {

template <int MT, int R, int S, int U>
hipError_t stream_instance(int64_t m, int64_t n, int64_t k, const void* aq, const float* as, const void* wq,
                           const float* ws, void* c, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_stream_kernel<MT, R, S, U>), dim3(stream_grid<R>(n)), dim3(64 * S), 0, stream,
                     static_cast<int>(m), n, k, static_cast<const unsigned char*>(aq), as,
                     static_cast<const unsigned char*>(wq), ws, static_cast<unsigned short*>(c));
  return hipGetLastError();
}

__global__ void fill_zero_kernel(unsigned short* __restrict__ c, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) c[i] = 0;
}

}  // namespace

// M-range dispatch of the streaming kernel: the token tile is the smallest
// MFMA multiple covering M, so every M in a range runs the same instruction
// stream (cost flat in M within the range).
hipError_t launch_gemm_stream(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                              const void* wq, const float* ws, void* c, hipStream_t stream) {
  if (m <= 16) return stream_instance<16, 1, 8, 4>(m, n, k, aq, as, wq, ws, c, stream);
  if (m <= 32) return stream_instance<32, 1, 8, 4>(m, n, k, aq, as, wq, ws, c, stream);
  return stream_instance<64, 1, 8, 2>(m, n, k, aq, as, wq, ws, c, stream);
}

hipError_t launch_gemm_tiled(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                             const void* wq, const float* ws, void* c, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const int64_t n_tiles = (n + BN - 1) / BN;
  const int64_t m_tiles = (m + BM - 1) / BM;
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN>), dim3(static_cast<unsigned>(n_tiles * m_tiles)), dim3(256), 0,
                     stream, m, n, k,
                     static_cast<const unsigned char*>(aq), as, static_cast<const unsigned char*>(wq), ws,
                     static_cast<unsigned short*>(c));
  return hipGetLastError();
}

hipError_t launch_fill_zero_bf16(int64_t count, void* c, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  blocks = blocks < 65536 ? blocks : 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<unsigned short*>(c), count);
  return hipGetLastError();
}

}  // namespace fp8bq
