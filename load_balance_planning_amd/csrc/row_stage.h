// A thread's share of a row of 16-byte vectors, staged through LDS, for the
// row copies of 256-thread workgroups (the dispatch gather, the deduplicated
// gather).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// Vectors c0, c0 + 256, ..., VPT of them (VPT <= 4), each only where it lies
// below `lim`, kept in the workgroup's LDS `s` ([VPT][256] vectors, this
// thread's at s[u * 256 + threadIdx.x]).  Each vector is written to LDS as its
// load returns, before the next load is issued, so a thread has one row load
// in flight.  Measured on MI355X at 8 resident workgroups per CU: the k-fold
// row copy runs faster this way than with all of a thread's loads in flight
// in registers (by 5-6 % on the DeepSeek-V3-sized gather), and faster than
// registers with each load awaited in turn (by 1-2 %).  (Up to VPT = 1 below.)
template <int VPT>
struct RowStage {
  static_assert(VPT >= 1 && VPT <= 4, "one to four vectors per thread");
  uint4* s;

  __device__ __forceinline__ void load(const uint4* __restrict__ src, int c0, int lim) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < VPT; ++u)
      if (c0 + u * 256 < lim) s[u * 256 + tid] = src[c0 + u * 256];
  }

  __device__ __forceinline__ void store(uint4* __restrict__ dst, int c0, int lim) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < VPT; ++u)
      if (c0 + u * 256 < lim) dst[c0 + u * 256] = s[u * 256 + tid];
  }
};

// One vector per thread: nothing to order, so it stays in a register (a
// clang vector: a uint4 member would keep the object in memory).
template <>
struct RowStage<1> {
  using vec16 = uint32_t __attribute__((ext_vector_type(4)));
  uint4* s;  // unused
  vec16 x;

  __device__ __forceinline__ void load(const uint4* __restrict__ src, int c0, int lim) {
    if (c0 < lim) x = reinterpret_cast<const vec16*>(src)[c0];
  }

  __device__ __forceinline__ void store(uint4* __restrict__ dst, int c0, int lim) const {
    if (c0 < lim) reinterpret_cast<vec16*>(dst)[c0] = x;
  }
};

}  // namespace moe
