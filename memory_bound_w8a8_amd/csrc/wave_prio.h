// Wave priority for the instruction arbiter of a SIMD (s_setprio, 0..3).
//
// Two waves share each SIMD in the 8-wave kernels. Left at equal priority
// they take the matrix core in age order: the older wave runs ahead and the
// younger one finishes its share alone, while the older waits at the next
// workgroup barrier. Lowering a wave's priority as it advances through its
// work (3 at the start, 0 near the end) prefers whichever wave is behind.
#pragma once

#include <hip/hip_runtime.h>

namespace fp8bq {

__device__ __forceinline__ void set_prio(int level) {
  switch (level) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

}  // namespace fp8bq
