// Two-stage vocabulary scoring on gfx950: exact top-k of the coarse bf16
// logits, then exact bf16 rescoring of the survivors.
//
// Page 1 (SmartX blog, "Qwen3.8-27B performance optimisation"), section
// "single-stream optimisation": the draft head reads the whole vocabulary
// projection every step; screening all candidates with FP8 scores and scoring
// only the survivors exactly in BF16 cuts that traffic. The coarse logits
// come from the block-FP8 GEMM (fp8bq_gemm / fp8bq_gemm_fused); this file
// holds the selection and the rescoring.
//
// Order: a bf16 value's 16-bit key is its bit pattern mapped to a monotone
// unsigned order (negative patterns inverted, positive ones with the top bit
// set, so -0 sits just below +0); entries compare by key, equal keys by the
// lower index. Packed with the inverted index below the key, every entry of a
// row is a distinct unsigned word, so selecting the largest words is exact
// and deterministic, and the value 0 (below every packed entry) pads.
//
// Top-k uses the bitonic top-k network (Shanbhag, Pirk, Madden, "Efficient
// Top-K Query Processing on Massively Parallel Hardware", SIGMOD 2018): with
// p the power of two >= k, sort segments of p with alternating directions,
// then repeatedly keep the element-wise maximum of each (ascending,
// descending) pair of segments -- the bitonic half-cleaner step, which holds
// the top p of the pair -- and bitonic-merge it, until one segment of p
// remains. Every step is a fixed compare-exchange pattern in LDS: no atomics,
// no data-dependent control flow, and far fewer stages than a full sort.
//   launch 1: a workgroup per 4096-logit chunk of a row writes the chunk's
//             top k as 64-bit words (key << 32 | ~index) to the workspace;
//   launch 2+: a workgroup per 4096 / p such lists merges them into one;
//             repeated until each row has one list, written as indices and
//             bf16 values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace fp8bq {

namespace {

constexpr int kChunk = 4096;          // logits per first-level workgroup
constexpr int kChunkThreads = 1024;
constexpr int kMergeEntries = 4096;   // 64-bit entries per merge workgroup (32 KiB LDS)
constexpr int kMergeThreads = 512;

__device__ __forceinline__ unsigned key16(unsigned b) { return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u); }
__device__ __forceinline__ unsigned unkey16(unsigned key) { return (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu); }

template <typename T>
__device__ __forceinline__ void compare_exchange(T* a, int lo, int hi, bool up) {
  const T x = a[lo], y = a[hi];
  if ((x > y) == up) {
    a[lo] = y;
    a[hi] = x;
  }
}

// Leaves the p largest of a[0 .. e) in a[0 .. p), in descending order.
// e and p are powers of two with e >= 2 p; entries are distinct or padding.
// The whole block calls it; it ends with a barrier.
template <typename T>
__device__ void bitonic_top(T* a, int e, int p, int log_p) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  __syncthreads();
  // sort every segment of p: even segments ascending, odd ones descending
  for (int size = 2; size <= p; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < e / 2; i += nt) {
        const int lo = 2 * i - (i & (stride - 1));
        compare_exchange(a, lo, lo + stride, (lo & size) == 0);
      }
      __syncthreads();
    }
  }
  // halve: segments sit gap apart; the pair (2j, 2j + 1) becomes segment j
  // at offset 2 j gap, merged ascending for even j and descending for odd j
  // (descending on the last level)
  for (int gap = p; gap < e; gap <<= 1) {
    const int pairs = e / (2 * gap);
    for (int i = tid; i < pairs * p; i += nt) {
      const int lo = 2 * (i >> log_p) * gap + (i & (p - 1));
      const T x = a[lo], y = a[lo + gap];
      a[lo] = x > y ? x : y;
    }
    __syncthreads();
    const int half = p >> 1;
    for (int stride = half; stride > 0; stride >>= 1) {
      for (int i = tid; i < pairs * half; i += nt) {
        const int j = i >> (log_p - 1);
        const int t = i & (half - 1);
        const int lo = 2 * j * gap + 2 * t - (t & (stride - 1));
        compare_exchange(a, lo, lo + stride, pairs > 1 && (j & 1) == 0);
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(int64_t v, int k, int p, int log_p, int chunks,
                                                                   const unsigned short* __restrict__ logits,
                                                                   unsigned long long* __restrict__ lists) {
  __shared__ unsigned buf[kChunk];
  const int64_t row = blockIdx.x / chunks;
  const int chunk = static_cast<int>(blockIdx.x - row * chunks);
  const int64_t base = static_cast<int64_t>(chunk) * kChunk;
  const unsigned short* x = logits + row * v;
  for (int i = threadIdx.x; i < kChunk; i += kChunkThreads) {
    const int64_t gi = base + i;
    buf[i] = gi < v ? (key16(x[gi]) << 16) | (0xffffu - static_cast<unsigned>(i)) : 0u;
  }
  bitonic_top(buf, kChunk, p, log_p);
  unsigned long long* out = lists + (row * chunks + chunk) * k;
  for (int j = threadIdx.x; j < k; j += kChunkThreads) {
    const unsigned w = buf[j];
    const unsigned gi = static_cast<unsigned>(base) + (0xffffu - (w & 0xffffu));
    out[j] = w == 0u ? 0ull : (static_cast<unsigned long long>(w >> 16) << 32) | (0xffffffffu - gi);
  }
}

// Merges `lists` sorted lists of k per row, `fan` lists per workgroup.
// Writes `lists_out` = ceil(lists / fan) lists per row to `next`, or, when
// that is 1, the row's final indices and values.
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(int k, int p, int log_p, int lists, int fan,
                                                                   const unsigned long long* __restrict__ src,
                                                                   unsigned long long* __restrict__ next,
                                                                   int* __restrict__ out_idx,
                                                                   unsigned short* __restrict__ out_val) {
  __shared__ unsigned long long buf[kMergeEntries];
  const int lists_out = (lists + fan - 1) / fan;
  const int64_t row = blockIdx.x / lists_out;
  const int part = static_cast<int>(blockIdx.x - row * lists_out);
  const int first = part * fan;
  const int count = lists - first < fan ? lists - first : fan;
  int segs = 2;
  while (segs < count) segs <<= 1;
  const int e = segs * p;
  const unsigned long long* in = src + (row * lists + first) * k;
  // list f lands in segment f: reversed (ascending) for even f, as is
  // (descending) for odd f, padded with 0 to p entries
  for (int i = threadIdx.x; i < e; i += kMergeThreads) {
    const int f = i >> log_p;
    const int s = i & (p - 1);
    const int j = (f & 1) ? s : p - 1 - s;
    buf[i] = (f < count && j < k) ? in[static_cast<int64_t>(f) * k + j] : 0ull;
  }
  bitonic_top(buf, e, p, log_p);
  if (lists_out > 1) {
    unsigned long long* out = next + (row * lists_out + part) * k;
    for (int j = threadIdx.x; j < k; j += kMergeThreads) out[j] = buf[j];
  } else {
    for (int j = threadIdx.x; j < k; j += kMergeThreads) {
      const unsigned long long w = buf[j];
      out_idx[row * k + j] = static_cast<int>(0xffffffffu - static_cast<unsigned>(w));
      out_val[row * k + j] = static_cast<unsigned short>(unkey16(static_cast<unsigned>(w >> 32)));
    }
  }
}

// Exact rescoring: wave w of workgroup (row, b) scores survivor 16 b + w.
// Lane l multiplies the bf16 pairs of the 16-byte pieces l, l + 64, ... of
// the two K rows (products exact in fp32), accumulating in fp32 in that
// order, element by element; the 64 lane sums are then added by xor
// butterflies (distance 32, 16, ..., 1). A survivor index outside [0, V)
// reads nothing and scores NaN.
constexpr int kRescoreWaves = 16;

__device__ __forceinline__ float bf16_lo_f(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_f(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float dot8(v4u a, v4u b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(bf16_lo_f(a[i]), bf16_lo_f(b[i]), acc);
    acc = fmaf(bf16_hi_f(a[i]), bf16_hi_f(b[i]), acc);
  }
  return acc;
}

__global__ __launch_bounds__(64 * kRescoreWaves) void rescore_kernel(int64_t kdim, int64_t v, int k, int blocks_per_row,
                                                                     const unsigned short* __restrict__ h,
                                                                     const unsigned short* __restrict__ w,
                                                                     const int* __restrict__ idx,
                                                                     float* __restrict__ scores) {
  const int64_t row = blockIdx.x / blocks_per_row;
  const int b = static_cast<int>(blockIdx.x - row * blocks_per_row);
  const int lane = threadIdx.x & 63;
  const int j = b * kRescoreWaves + (threadIdx.x >> 6);
  if (j >= k) return;
  const int r = idx[row * k + j];
  if (r < 0 || r >= v) {
    if (lane == 0) scores[row * k + j] = __builtin_nanf("");
    return;
  }
  const v4u* hrow = reinterpret_cast<const v4u*>(h + row * kdim);
  const v4u* wrow = reinterpret_cast<const v4u*>(w + static_cast<int64_t>(r) * kdim);
  const int64_t pieces = kdim >> 3;
  float acc = 0.f;
#pragma unroll 8
  for (int64_t i = lane; i < pieces; i += 64) acc = dot8(hrow[i], __builtin_nontemporal_load(wrow + i), acc);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) scores[row * k + j] = acc;
}

// Best survivor of each row by (score descending, index ascending); NaN
// scores never win; -1 when every score is NaN. One wave per row.
__global__ __launch_bounds__(64) void pick_kernel(int k, const int* __restrict__ idx, const float* __restrict__ scores,
                                                  int* __restrict__ pick) {
  const int64_t row = blockIdx.x;
  float best = 0.f;
  int bi = -1;
  for (int j = threadIdx.x; j < k; j += 64) {
    const float s = scores[row * k + j];
    const int r = idx[row * k + j];
    if (s == s && (bi < 0 || s > best || (s == best && r < bi))) {
      best = s;
      bi = r;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float s = __shfl_xor(best, off);
    const int r = __shfl_xor(bi, off);
    if (r >= 0 && (bi < 0 || s > best || (s == best && r < bi))) {
      best = s;
      bi = r;
    }
  }
  if (threadIdx.x == 0) pick[row] = bi;
}

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

int log2_exact(int p) { return __builtin_ctz(static_cast<unsigned>(p)); }

int64_t chunks_of(int64_t v) { return (v + kChunk - 1) / kChunk; }

}  // namespace

int64_t topk_workspace_bytes(int64_t m, int64_t v, int64_t k) {
  const int64_t fan = kMergeEntries / pow2_at_least(static_cast<int>(k));
  const int64_t l0 = chunks_of(v);
  const int64_t l1 = (l0 + fan - 1) / fan;
  return (l0 + l1) * m * k * static_cast<int64_t>(sizeof(unsigned long long));
}

int64_t topk_grid_blocks(int64_t m, int64_t v) { return m * chunks_of(v); }

hipError_t launch_topk(int64_t m, int64_t v, int k, const void* logits, void* workspace, int* idx, void* val,
                       hipStream_t stream) {
  const int p = pow2_at_least(k);
  const int log_p = log2_exact(p);
  const int fan = kMergeEntries / p;
  int lists = static_cast<int>(chunks_of(v));
  auto* a = static_cast<unsigned long long*>(workspace);
  auto* b = a + static_cast<int64_t>(lists) * m * k;  // the second level's lists
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(static_cast<unsigned>(m * lists)), dim3(kChunkThreads), 0, stream, v, k,
                     p, log_p, lists, static_cast<const unsigned short*>(logits), a);
  hipError_t e = hipGetLastError();
  while (e == hipSuccess) {
    const int lists_out = (lists + fan - 1) / fan;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(m * lists_out)), dim3(kMergeThreads), 0, stream, k,
                       p, log_p, lists, fan, a, b, idx, static_cast<unsigned short*>(val));
    e = hipGetLastError();
    if (lists_out == 1) break;
    lists = lists_out;
    auto* t = a;
    a = b;
    b = t;
  }
  return e;
}

int64_t rescore_grid_blocks(int64_t m, int64_t k) { return m * ((k + kRescoreWaves - 1) / kRescoreWaves); }

hipError_t launch_rescore(int64_t m, int64_t kdim, int64_t v, int64_t k, const void* h, const void* w,
                          const int* idx, float* scores, int* pick, hipStream_t stream) {
  const int blocks_per_row = static_cast<int>((k + kRescoreWaves - 1) / kRescoreWaves);
  hipLaunchKernelGGL(rescore_kernel, dim3(static_cast<unsigned>(m * blocks_per_row)), dim3(64 * kRescoreWaves), 0,
                     stream, kdim, v, static_cast<int>(k), blocks_per_row, static_cast<const unsigned short*>(h),
                     static_cast<const unsigned short*>(w), idx, scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pick_kernel, dim3(static_cast<unsigned>(m)), dim3(64), 0, stream, static_cast<int>(k), idx, scores,
                     pick);
  return hipGetLastError();
}

}  // namespace fp8bq
