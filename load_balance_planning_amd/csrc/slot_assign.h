// The slot-to-instance assignment, shared by the assignment kernel and the
// assigning gather of the single-call step.
//
// Slot sigma = t*k + j of token t (source s, tile x, bit b of the tile) with
// expert e.  Its rank p among the slots of (s, e) in token order is the tile
// prefix plus the popcount of the mask bits below b.  An expert with one
// instance keeps all its slots there, at position tile_base + popcount (its
// segment lists the slots of every source in token order).  Otherwise the
// slot goes to the first instance (rank order) whose running quota sum of
// source s exceeds p, at that instance's column prefix plus the remainder
// ([TopoEP] section 4.3; the quota and slot rules of moe_plan.h).
#pragma once

#include "internal.h"

namespace moe {

__device__ __forceinline__ void assign_slot(const Dims& d, int64_t sigma, const int32_t* __restrict__ topk,
                                            const uint64_t* __restrict__ tile_mask,
                                            const int32_t* __restrict__ tile_base,
                                            const int32_t* __restrict__ quota, const Workspace& ws, int& inst,
                                            int& rank) {
  const int64_t t = sigma / d.k;
  const int s = (int)(t / d.Tr);
  const int tl = (int)(t - (int64_t)s * d.Tr);
  const int x = s * d.C + (tl >> 6);
  const int bit = tl & 63;
  const int e = topk[sigma];
  inst = -1;
  rank = -1;
  if ((unsigned)e < (unsigned)d.E) {
    const uint64_t m = tile_mask[(int64_t)x * d.E + e];
    const int low = __popcll(m & ((1ull << bit) - 1ull));
    const int base = tile_base[(int64_t)x * d.E + e];
    const int o0 = ws.einst_off[e], o1 = ws.einst_off[e + 1];
    if (o1 - o0 == 1) {
      inst = ws.einst_list[o0];
      rank = base + low;
    } else {
      const int p = base - tile_base[(int64_t)s * d.C * d.E + e] + low;
      int cum = 0;
      for (int a = o0; a < o1; ++a) {
        const int i = ws.einst_list[a];
        if ((unsigned)i >= (unsigned)d.cap) break;
        const int qv = quota[(int64_t)s * d.cap + i];
        if (p < cum + qv) {
          inst = i;
          rank = ws.colpre[(int64_t)i * d.R + s] + (p - cum);
          break;
        }
        cum += qv;
      }
    }
  }
  if (inst < 0) atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
}

}  // namespace moe
