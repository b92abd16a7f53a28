// Token-shuffle prediction on gfx950.
//
// [Coupling] "Moving Tokens Toward Their Next Experts": a token's experts at
// this layer predict the GPU that holds most of its next-layer experts, and
// the token is moved there before the next router runs.  Each of the token's
// experts a votes with its empirical next-layer distribution over ranks,
//   P[a][r]  = (sum over experts b on rank r of X[a][b]) / count[a]
//   score[r] = P[a_0][r] + ... + P[a_{k-1}][r]        (slot order, IEEE double)
//   pred     = argmax_r score[r], ties to the lower rank
// with X the layer-to-layer transition counts (moe_plan_route's trans of the
// next layer) and count this layer's expert counts.
//
// Two launches: one workgroup per expert a sums its transition row by
// destination rank in LDS (64-bit) and writes P[a][*] (E x R doubles, the
// handle's workspace); then a group of P lanes per token (P the power of two
// covering R, at most 64), lane r of the group holding ranks r, r+P, ...,
// adds its experts' rows in slot order and takes the argmax (largest score,
// then lowest rank, by two reductions over the group).  With the next layer's
// top-k the same group counts its slots on the predicted rank and on its own
// source rank (the locality with and without the shuffle).
#include "internal.h"

namespace moe {
namespace {

constexpr int kVoteThreads = 256;
constexpr int kPredThreads = 1024;
constexpr int kPredTokens = 64;  // tokens per workgroup

struct PredictArgs {
  const int32_t* cur;      // [T][k] this layer's top-k
  const int32_t* trans;    // [E][E] this layer -> next layer
  const int32_t* count;    // [E] this layer's expert counts
  const int32_t* rank_of;  // [E] rank of each next-layer expert, or null: b / Er
  const int32_t* next;     // [T][k] the next layer's top-k, or null
  double* vote;            // [E][R] workspace
  int32_t* pred;
  int32_t* rank_tokens;
  int64_t* local;          // [2], or null
  int32_t* status;
};

__device__ __forceinline__ int dest_rank(const Dims& d, const int32_t* rank_of, int b) {
  return rank_of ? rank_of[b] : b / d.Er;
}

__global__ __launch_bounds__(kVoteThreads) void vote_kernel(Dims d, PredictArgs pa) {
  __shared__ unsigned long long hist[kMaxR];
  const int a = blockIdx.x, tid = threadIdx.x;
  if (a == 0) {  // outputs accumulated by the prediction kernel start at zero
    for (int r = tid; r < d.R; r += kVoteThreads) pa.rank_tokens[r] = 0;
    if (pa.local && tid < 2) pa.local[tid] = 0;
  }
  for (int r = tid; r < d.R; r += kVoteThreads) hist[r] = 0;
  __syncthreads();
  bool bad_rank = false, bad_count = false;
  for (int b = tid; b < d.E; b += kVoteThreads) {
    const int r = dest_rank(d, pa.rank_of, b);
    const int32_t x = pa.trans[(int64_t)a * d.E + b];
    if ((unsigned)r >= (unsigned)d.R) {
      bad_rank = true;
      continue;
    }
    bad_count |= x < 0;
    if (x != 0) atomicAdd(&hist[r], (unsigned long long)(int64_t)x);
  }
  const int32_t c = pa.count[a];
  if (tid == 0) bad_count |= c < 0;
  if (bad_rank) atomicOr(pa.status, MOE_STATUS_BAD_KEY);
  if (bad_count) atomicOr(pa.status, MOE_STATUS_BAD_PAIRS);
  __syncthreads();
  for (int r = tid; r < d.R; r += kVoteThreads)
    pa.vote[(int64_t)a * d.R + r] = c > 0 ? (double)(int64_t)hist[r] / (double)c : 0.0;
}

// Order-preserving bits of a non-negative double (sums of votes are >= +0).
__device__ __forceinline__ uint64_t dbits(double x) { return (uint64_t)__double_as_longlong(x); }

template <int P>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int off = P / 2; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, P);
    v = o > v ? o : v;
  }
  return v;
}

template <int P>
__device__ __forceinline__ int group_min(int v) {
#pragma unroll
  for (int off = P / 2; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, P));
  return v;
}

template <int P>
__device__ __forceinline__ int group_sum(int v) {
#pragma unroll
  for (int off = P / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, P);
  return v;
}

// A group of P lanes (a power of two, P >= min(R, 64)) per token; lane l of
// the group holds ranks l, l + P, ... (RPL of them).  A workgroup of 1024
// threads takes kPredTokens consecutive tokens.
template <int P, int RPL>
__global__ __launch_bounds__(kPredThreads) void predict_kernel(Dims d, PredictArgs pa) {
  __shared__ int32_t hist[kMaxR];
  __shared__ int32_t loc[2];
  constexpr int kGroups = kPredThreads / P;
  const int tid = threadIdx.x, sub = tid % P, grp = tid / P;
  for (int r = tid; r < d.R; r += kPredThreads) hist[r] = 0;
  if (tid < 2) loc[tid] = 0;
  __syncthreads();
  bool bad = false;
  int hp = 0, hs = 0;
  for (int i = grp; i < kPredTokens; i += kGroups) {
    const int64_t t = (int64_t)blockIdx.x * kPredTokens + i;
    if (t >= d.T) break;  // uniform across the group
    double score[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) score[u] = 0.0;
    for (int j = 0; j < d.k; ++j) {
      const int a = pa.cur[t * d.k + j];
      if ((unsigned)a >= (unsigned)d.E) {
        bad = true;
        continue;
      }
      const double* row = pa.vote + (int64_t)a * d.R;
#pragma unroll
      for (int u = 0; u < RPL; ++u) {
        const int r = sub + P * u;
        if (r < d.R) score[u] += row[r];
      }
    }
    uint64_t best = 0;
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int r = sub + P * u;
      if (r < d.R) best = dbits(score[u]) > best ? dbits(score[u]) : best;
    }
    best = group_max_u64<P>(best);
    int br = INT32_MAX;
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int r = sub + P * u;
      if (r < d.R && dbits(score[u]) == best) br = min(br, r);
    }
    br = group_min<P>(br);
    if (sub == 0) {
      pa.pred[t] = br;
      atomicAdd(&hist[br], 1);
    }
    if (pa.next && pa.local) {
      for (int j = sub; j < d.k; j += P) {
        const int b = pa.next[t * d.k + j];
        if ((unsigned)b < (unsigned)d.E) {
          const int rb = dest_rank(d, pa.rank_of, b);
          hp += rb == br;
          hs += rb == (int)(t / d.Tr);
        } else {
          bad = true;
        }
      }
    }
  }
  if (bad) atomicOr(pa.status, MOE_STATUS_BAD_TOPK);
  if (pa.next && pa.local) {
    hp = group_sum<64>(hp);
    hs = group_sum<64>(hs);
    if ((tid & 63) == 0 && (hp | hs)) {
      atomicAdd(&loc[0], hp);
      atomicAdd(&loc[1], hs);
    }
  }
  __syncthreads();
  for (int r = tid; r < d.R; r += kPredThreads)
    if (hist[r]) atomicAdd(&pa.rank_tokens[r], hist[r]);
  if (pa.local && tid < 2 && loc[tid]) atomicAdd(reinterpret_cast<unsigned long long*>(&pa.local[tid]),
                                                 (unsigned long long)loc[tid]);
}

template <int P, int RPL>
void launch_pred(const Dims& d, const PredictArgs& pa, hipStream_t st) {
  hipLaunchKernelGGL((predict_kernel<P, RPL>), dim3((d.T + kPredTokens - 1) / kPredTokens), dim3(kPredThreads), 0,
                     st, d, pa);
}

}  // namespace

hipError_t launch_predict(const Dims& d, const int32_t* topk_cur, const int32_t* trans, const int32_t* count_cur,
                          const int32_t* key_rank, const int32_t* topk_next, const moe_predict_out& out,
                          const Workspace& ws, hipStream_t st) {
  const PredictArgs pa{topk_cur, trans, count_cur, key_rank, topk_next, ws.pred_vote,
                       out.pred, out.rank_tokens, out.local, ws.status};
  hipLaunchKernelGGL(vote_kernel, dim3(d.E), dim3(kVoteThreads), 0, st, d, pa);
  if (d.T > 0) {
    if (d.R <= 1) launch_pred<1, 1>(d, pa, st);
    else if (d.R <= 2) launch_pred<2, 1>(d, pa, st);
    else if (d.R <= 4) launch_pred<4, 1>(d, pa, st);
    else if (d.R <= 8) launch_pred<8, 1>(d, pa, st);
    else if (d.R <= 16) launch_pred<16, 1>(d, pa, st);
    else if (d.R <= 32) launch_pred<32, 1>(d, pa, st);
    else if (d.R <= 64) launch_pred<64, 1>(d, pa, st);
    else if (d.R <= 128) launch_pred<64, 2>(d, pa, st);
    else launch_pred<64, kMaxR / 64>(d, pa, st);
  }
  return hipGetLastError();
}

}  // namespace moe
