// Gate-weighted combine on gfx950: the return path of the dispatch.
//
// [TopoEP] section 2.1, Fig. 1: after the experts, each token's k expert
// outputs come back and are summed.  The gate weights are the softmax of the
// token's k selected logits (the maximum taken out before exp):
//   w[t][j]   = exp(v[t][j] - max) / sum_j' exp(v[t][j'] - max)
//   out[t][:] = bf16( sum over j = 0..k-1 of w[t][j] * expert_out[slot_pos[t*k+j]][:] )
// accumulated in fp32 in slot order and rounded once to bf16 (nearest even).
//
// One workgroup per token: the first wave computes the weights and reads the
// k row positions into LDS; every thread then owns 32 columns (four 16-byte
// vectors) and streams the k rows through them, eight rows' loads in flight.
// HBM traffic is k rows read and one written per token -- the mirror of the
// gather.  The expert rows are read once, with non-temporal loads (measured
// on MI355X: DeepSeek-V3-shaped layer 798 -> 777 us, Kimi-K2-shaped 757 ->
// 712 us).
#include "internal.h"

namespace moe {
namespace {

constexpr int kCombThreads = 256;
constexpr int kRowsInFlight = 8;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// acc[0..7] += w * (8 bf16 values of v), each an fp32 FMA.
__device__ __forceinline__ void fma_row(float* acc, float w, const uint4& v) {
  acc[0] = fmaf(w, bf16_lo(v.x), acc[0]);
  acc[1] = fmaf(w, bf16_hi(v.x), acc[1]);
  acc[2] = fmaf(w, bf16_lo(v.y), acc[2]);
  acc[3] = fmaf(w, bf16_hi(v.y), acc[3]);
  acc[4] = fmaf(w, bf16_lo(v.z), acc[4]);
  acc[5] = fmaf(w, bf16_hi(v.z), acc[5]);
  acc[6] = fmaf(w, bf16_lo(v.w), acc[6]);
  acc[7] = fmaf(w, bf16_hi(v.w), acc[7]);
}

// Weights and row positions of token t into LDS (first wave).  A non-finite
// selected logit or a position outside the dispatch buffer is recorded in the
// status word; such a position is stored as -1 and its slot skipped.
__device__ __forceinline__ void gate_weights(const Dims& d, int64_t t, const float* __restrict__ topk_val,
                                             const int32_t* __restrict__ slot_pos, float* w_s, int32_t* p_s,
                                             int32_t* status) {
  const int lane = threadIdx.x;
  if (lane < 64) {
    const bool on = lane < d.k;
    const float v = on ? topk_val[t * d.k + lane] : -INFINITY;
    if (on && !__builtin_isfinite(v)) atomicOr(status, MOE_STATUS_NAN_LOGIT);
    float m = v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float e = on ? expf(v - m) : 0.0f;
    float s = e;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (on) {
      w_s[lane] = e / s;
      int32_t p = slot_pos[t * d.k + lane];
      const int64_t N = (int64_t)d.T * d.k;
      if (p < 0 || p >= N) {
        atomicOr(status, MOE_STATUS_PLAN_CHECK);
        p = -1;
      }
      p_s[lane] = p;
    }
  }
  __syncthreads();
}

template <int VPT>
__global__ __launch_bounds__(kCombThreads) void combine_vec_kernel(Dims d, const float* __restrict__ topk_val,
                                                                   const int32_t* __restrict__ slot_pos,
                                                                   const uint4* __restrict__ expert_out,
                                                                   uint4* __restrict__ out, int32_t* __restrict__ status) {
  __shared__ float w_s[kMaxK];
  __shared__ int32_t p_s[kMaxK];
  const int64_t t = blockIdx.x;
  gate_weights(d, t, topk_val, slot_pos, w_s, p_s, status);
  const int vpr = d.H / 8;
  for (int base = 0; base < vpr; base += kCombThreads * VPT) {
    float acc[VPT][8];
#pragma unroll
    for (int u = 0; u < VPT; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    // kRowsInFlight rows loaded per batch (measured on MI355X: 8 beats 2 and 4
    // by ~5 %, more rows cost occupancy); the sums still go j = 0, 1, 2, ... in order
    for (int j = 0; j < d.k; j += kRowsInFlight) {
      int pj[kRowsInFlight];
      float wj[kRowsInFlight];
#pragma unroll
      for (int q = 0; q < kRowsInFlight; ++q) {
        pj[q] = j + q < d.k ? p_s[j + q] : -1;
        wj[q] = pj[q] >= 0 ? w_s[j + q] : 0.0f;
      }
      uint4 x[kRowsInFlight][VPT];
#pragma unroll
      for (int q = 0; q < kRowsInFlight; ++q) {
        const uint4* row = expert_out + (int64_t)(pj[q] >= 0 ? pj[q] : 0) * vpr;
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int c = base + threadIdx.x + u * kCombThreads;
          const v4u y = c < vpr && pj[q] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(row) + c)
                                              : v4u{0, 0, 0, 0};  // a skipped slot adds 0 * 0
          x[q][u] = make_uint4(y.x, y.y, y.z, y.w);
        }
      }
#pragma unroll
      for (int q = 0; q < kRowsInFlight; ++q)
        if (j + q < d.k)
#pragma unroll
          for (int u = 0; u < VPT; ++u) fma_row(acc[u], wj[q], x[q][u]);
    }
    uint4* dst = out + t * vpr;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = base + threadIdx.x + u * kCombThreads;
      if (c < vpr) {
        uint4 y;
        y.x = to_bf16(acc[u][0]) | (to_bf16(acc[u][1]) << 16);
        y.y = to_bf16(acc[u][2]) | (to_bf16(acc[u][3]) << 16);
        y.z = to_bf16(acc[u][4]) | (to_bf16(acc[u][5]) << 16);
        y.w = to_bf16(acc[u][6]) | (to_bf16(acc[u][7]) << 16);
        dst[c] = y;
      }
    }
  }
}

// Any H: one bf16 element per thread and step.
__global__ __launch_bounds__(kCombThreads) void combine_u16_kernel(Dims d, const float* __restrict__ topk_val,
                                                                   const int32_t* __restrict__ slot_pos,
                                                                   const uint16_t* __restrict__ expert_out,
                                                                   uint16_t* __restrict__ out,
                                                                   int32_t* __restrict__ status) {
  __shared__ float w_s[kMaxK];
  __shared__ int32_t p_s[kMaxK];
  const int64_t t = blockIdx.x;
  gate_weights(d, t, topk_val, slot_pos, w_s, p_s, status);
  for (int c = threadIdx.x; c < d.H; c += kCombThreads) {
    float acc = 0.0f;
    for (int j = 0; j < d.k; ++j) {
      const int p = p_s[j];
      if (p >= 0) acc = fmaf(w_s[j], __uint_as_float((uint32_t)expert_out[(int64_t)p * d.H + c] << 16), acc);
    }
    out[t * d.H + c] = (uint16_t)to_bf16(acc);
  }
}

}  // namespace

hipError_t launch_combine(const Dims& d, const float* topk_val, const int32_t* slot_pos, const uint16_t* expert_out,
                          uint16_t* out, int32_t* status, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  const bool vec = (d.H % 8) == 0 && ((uintptr_t)expert_out % 16) == 0 && ((uintptr_t)out % 16) == 0;
  if (vec) {
    // a row of at most kCombThreads vectors takes one round: no dead registers
    if (d.H / 8 <= kCombThreads)
      hipLaunchKernelGGL((combine_vec_kernel<1>), dim3(d.T), dim3(kCombThreads), 0, st, d, topk_val, slot_pos,
                         reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(out), status);
    else
      hipLaunchKernelGGL((combine_vec_kernel<4>), dim3(d.T), dim3(kCombThreads), 0, st, d, topk_val, slot_pos,
                         reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(out), status);
  } else {
    hipLaunchKernelGGL(combine_u16_kernel, dim3(d.T), dim3(kCombThreads), 0, st, d, topk_val, slot_pos, expert_out,
                       out, status);
  }
  return hipGetLastError();
}

}  // namespace moe
