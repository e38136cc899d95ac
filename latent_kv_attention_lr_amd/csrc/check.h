// check.h -- internal: the bounds test of the checked build.
//
// Built with LR_ATTN_CHECK = 1 (liblr_attn_check.so), the kernels pass every
// address of a cache, workspace, weight, input or output access through
// checked(): one outside the buffer's extent is counted in the device
// counter of its translation unit and redirected to the buffer's first bytes,
// so the launch completes and the host reads the count (lr_attn_check_count)
// instead of a fault.  In the release build checked() returns its argument.
#pragma once

#include <stdint.h>

#ifndef LR_ATTN_CHECK
#define LR_ATTN_CHECK 0
#endif

namespace lr {

struct Bounds {
  const uint8_t* lo;   // the buffer
  uint64_t n;          // its bytes
};

#if LR_ATTN_CHECK
// one per translation unit (internal linkage) and per device
static __device__ unsigned long long g_check_count;
#endif

template <typename P>
__device__ __forceinline__ P checked(const Bounds& bd, P p, int bytes) {
#if LR_ATTN_CHECK
  const uint8_t* q = reinterpret_cast<const uint8_t*>(p);
  if (q < bd.lo || q + bytes > bd.lo + bd.n) {
    atomicAdd(&g_check_count, 1ull);
    return reinterpret_cast<P>(const_cast<uint8_t*>(bd.lo));
  }
#else
  (void)bd;
  (void)bytes;
#endif
  return p;
}

}  // namespace lr
