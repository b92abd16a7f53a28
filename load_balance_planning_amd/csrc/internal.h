// Internal declarations of the moe_plan HIP library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_plan.h"

namespace moe {

// Limits of the library (checked by moe_plan_create).
constexpr int kMaxE = 2048;
constexpr int kMaxK = 32;
constexpr int kMaxR = 256;
constexpr int kMaxG = 64;
constexpr int kMaxB = 1024;
constexpr int kTile = 64;  // tokens per tile: one bit per token in a 64-bit presence mask

// LDS of one CU, the block size in which it is given to a workgroup, and the
// LDS of one workgroup of the row copy (its row staged as four 16-byte
// vectors per thread of 256, plus the k slot positions, in whole blocks).
// The copy keeps eight workgroups resident per CU; a workgroup of another
// launch is placed beside them only when it asks for at most what they leave
// free, so the launches meant to run beside another batch's row copy (top-k,
// solver, quotas) keep each workgroup's whole LDS, static and dynamic,
// within kBesideGatherLds.
constexpr size_t kCuLdsBytes = 160 * 1024;
constexpr size_t kLdsBlock = 512;
constexpr size_t kGatherWgLds = (4 * 256 * 16 + 4 * kMaxK + kLdsBlock - 1) / kLdsBlock * kLdsBlock;
constexpr size_t kBesideGatherLds = kCuLdsBytes - 8 * kGatherWgLds;

// Everything a kernel needs to know about the layer, derived once at create time.
struct Dims {
  int32_t T, E, k, R, G, H, B;
  int32_t M;        // domains
  int32_t Tr;       // tokens per source rank
  int32_t Er;       // experts per rank (main instances)
  int32_t C;        // tiles per source rank
  int32_t NT;       // tiles
  int32_t cap;      // instance capacity E + B
  int32_t n_slot;   // replica slots per rank
  int32_t max_iters;
  int64_t S, W;     // token bytes, expert bytes
};

// Device workspace owned by a handle.
struct Workspace {
  int32_t* status;      // [1]   MOE_STATUS_* bits
  uint64_t* tile_mask;  // [NT][E] presence masks of the top-k: bit j of [x][e] is set when
                        // token j of tile x selects e (tile x = s*C + c: tokens s*Tr + 64c ...)
  int32_t* tile_base;   // [NT][E] assignments of e in all earlier tiles (exclusive prefix)
  uint64_t* prev_mask;  // [NT][E] presence masks of the previous layer's top-k
  int32_t* demand;      // [M][E] domain demand D (Eq. 4) when it does not fit in LDS
  int32_t* einst_off;   // [E+1] per-expert instance lists (rank order) ...
  int32_t* einst_list;  // [cap] ... instance ids
  int32_t* rlist;       // [E+1] experts with more than one instance; entry E is their count
  int32_t* colpre;      // [cap][R] exclusive prefix of each instance's quotas over sources
  int32_t* pair_part;   // partial pair-count blocks of the tile splits (pair_part_words)
  int32_t* omega_acc;   // [R][E] routing matrix accumulated by the top-k kernel of
                        // moe_plan_step; zero between calls (the slot assignment clears it)
  int32_t* place_aff;   // [R][E] placement affinities
  uint64_t* place_key;  // [R][R] best swap key per rank pair
  int32_t* place_int;   // [4][E] placement: degrees, largest entry per row, rank of each expert, own affinity
  int32_t* place_mem;   // [E] placement: the experts of each rank, E/R per rank
  uint16_t* place_c16;  // [place_c16_elems] 16-bit copy of the co-selection counts
  uint64_t* dd_mask;    // [NT][R] deduplication: tokens of each tile with a slot on each rank
  int32_t* dd_cnt;      // [NT][R] slots of each tile on each rank
  int32_t* dd_base;     // [NT][R] rows of each rank before each tile
  int32_t* dd_count;    // [R] rows of each rank
  double* pred_vote;    // [E][R] token-shuffle votes: each expert's next-layer share per rank
};

// Pair-count job: presence masks in, co-selection / transition blocks out
// (pair_count.h).  nz slices starting at zbase: 0 co-selection, 1 transitions.
struct PairArgs {
  const uint64_t* cur;   // this layer's masks
  const uint64_t* prev;  // the previous layer's masks (transitions)
  int32_t* cooc;
  int32_t* trans;
  int32_t* part;         // split partials (workspace)
  int splits, nz, zbase;
};
PairArgs pair_args(const Dims& d, const uint64_t* tile_mask, const uint64_t* prev_mask, int32_t* cooc, int32_t* trans,
                   int32_t* part, int nthr);
// The scan of launch_scan and the pair counts of the masks (cooc, and trans
// from prev_mask; nullable) in one launch plus the pairs' reduction, on `st`.
hipError_t launch_scan_pairs(const Dims& d, const uint64_t* tile_mask, int32_t* tile_base, int32_t* omega,
                             int32_t* count, const uint64_t* prev_mask, int32_t* cooc, int32_t* trans, int32_t* part,
                             hipStream_t st);

// The per-tile histogram scan (tile_scan.h) run by extra workgroups of the
// solver launch: from the masks, the tile prefix into base and, each when
// non-null, the routing matrix and expert counts into omega / count, and a
// comparison of the routing matrix with `check` (MOE_STATUS_BAD_OMEGA on a
// difference).
struct ScanJob {
  const uint64_t* mask;
  int32_t* base;
  int32_t* omega;
  int32_t* count;
  const int32_t* check;
};

// Validates a configuration and derives the dimensions (moe_plan_create's checks).
int derive_dims(const moe_plan_config* c, Dims* d);
// Argument checks of moe_plan_step (MOE_OK or MOE_ERR_INVALID_ARG).
int check_step_args(const Dims& d, const float* logits, const uint16_t* hidden, const moe_route_out* route,
                    const moe_plan_out* plan, const moe_dispatch_out* out);
struct KernelEvents;
// The launches of moe_plan_step on `st` (ws.omega_acc must be zero on entry;
// it is zero again when the work ends).
hipError_t enqueue_step(const Dims& d, const Workspace& ws, const float* logits, const int32_t* prev_topk,
                        const uint16_t* hidden, const moe_route_out& route, const moe_plan_out& plan,
                        const moe_dispatch_out& out, const KernelEvents& ev, hipStream_t st);

// Launchers (all asynchronous on `st`).
// omega_acc (nullable): also add each tile's per-expert counts to this [R][E]
// accumulator (which must be zero on entry).
hipError_t launch_route_topk(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                             float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* omega_acc,
                             int32_t* status, hipStream_t st);
hipError_t launch_build_masks(const Dims& d, const int32_t* topk_idx, const int32_t* prev_topk,
                              uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status, hipStream_t st);
// omega / count nullable: then only the tile prefix is written.
hipError_t launch_scan(const Dims& d, const uint64_t* tile_mask, int32_t* tile_base, int32_t* omega,
                       int32_t* count, hipStream_t st);
// Solver and quotas from the routing matrix omega.  When scan.mask is given,
// extra workgroups of the solver launch run the scan job, and the pair counts
// of those masks (and of prev_mask) go to cooc / trans, reduced by extra
// workgroups of the quota launch (each output nullable; part: workspace).
// With inst_offset / rank_offset non-null the quota launch also writes the
// dispatch offsets of the plan.  beside: the solver launch is to run beside
// another batch's row copy (256-thread workgroups within kBesideGatherLds of
// LDS) rather than alone (512-thread workgroups); the outputs are the same.
hipError_t launch_plan(const Dims& d, const int32_t* omega, const ScanJob& scan, const uint64_t* prev_mask,
                       int32_t* cooc, int32_t* trans, int32_t* part, const moe_plan_out& out, int32_t* inst_offset,
                       int32_t* rank_offset, const Workspace& ws, bool beside, hipStream_t st);
// Zero n int32 words (a fill kernel: safe inside graph capture).
hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t st);
// The slot assignment; it also zeroes clear[0, clear_n) (nullable), which no
// kernel before it on the stream still reads.
hipError_t launch_assign(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                         const int32_t* tile_base, const moe_plan_out& out, const Workspace& ws,
                         int32_t* clear, int64_t clear_n, hipStream_t st);
// The dispatch of a plan: its offsets (into inst_offset / rank_offset) and the
// gather at slot_pos = inst_offset[slot_inst] + slot_rank, in one launch.
// Events around a gather kernel's launch (each nullable): `wait` is waited
// for on the stream right before the launch, `begin` / `end` are recorded
// right before and after it (timing), `done` right after it (ordering).
struct KernelEvents {
  hipEvent_t begin;
  hipEvent_t end;
  hipEvent_t wait;
  hipEvent_t done;
};
// Whether these hooks order the row copy with another handle's (a batch
// pipelined beside another): the solver launch is then sized to be placed
// beside that handle's running copy.
inline bool pipelined(const KernelEvents& ev) { return ev.wait != nullptr || ev.done != nullptr; }
// The launch of a gather kernel between the hooks of `ev`.
hipError_t gather_hooks_before(const KernelEvents& ev, hipStream_t st);
hipError_t gather_hooks_after(const KernelEvents& ev, hipStream_t st);
hipError_t launch_gather(const Dims& d, const moe_plan_out& plan, const uint16_t* hidden, int32_t* perm,
                         int32_t* slot_pos, int32_t* inst_offset, int32_t* rank_offset, uint16_t* dispatch,
                         const Workspace& ws, const KernelEvents& ev, hipStream_t st);
// The row copy alone (no dispatch offsets) from the plan's slot_inst / slot_rank.
hipError_t launch_gather_rows(const Dims& d, const moe_plan_out& plan, const uint16_t* hidden, int32_t* perm,
                              int32_t* slot_pos, const int32_t* inst_offset, uint16_t* dispatch, const Workspace& ws,
                              const KernelEvents& ev, hipStream_t st);
// The gather that also assigns the slots (writes plan.slot_inst / slot_rank),
// one workgroup per token; only for 16-byte-aligned rows with H a multiple of
// 8 (gather_can_assign).  The single call uses it where the copy runs in one
// part per token (copy_in_one_part); elsewhere it assigns first and copies in
// parts, since each part would repeat the assignment's dependent loads.
bool gather_can_assign(const Dims& d, const uint16_t* hidden, const uint16_t* dispatch);
bool copy_in_one_part(const Dims& d);
hipError_t launch_assign_gather(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                                const int32_t* tile_base, const moe_plan_out& plan, const int32_t* inst_offset,
                                const uint16_t* hidden, int32_t* perm, int32_t* slot_pos, uint16_t* dispatch,
                                const Workspace& ws, int32_t* clear, int64_t clear_n, const KernelEvents& ev,
                                hipStream_t st);

hipError_t launch_combine(const Dims& d, const float* topk_val, const int32_t* slot_pos, const uint16_t* expert_out,
                          uint16_t* out, int32_t* status, hipStream_t st);

// Correlated placement (one workgroup) from co-selection counts.
hipError_t launch_place(const Dims& d, const int32_t* cooc, int32_t max_swaps, const moe_place_out& out,
                        const Workspace& ws, hipStream_t st);
// Deduplicated counts; with hidden non-null also the layout and row copy.
hipError_t launch_dedup(const Dims& d, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                        const uint16_t* hidden, const moe_dedup_out& out, const Workspace& ws, hipStream_t st);

// Plan-quality counters (int64 [8]) from a plan's quotas, instances and loads.
hipError_t launch_quality(const Dims& d, const moe_plan_out& plan, int64_t* out, int32_t* status, hipStream_t st);

// Token-shuffle prediction from the layer-to-layer transition counts.
hipError_t launch_predict(const Dims& d, const int32_t* topk_cur, const int32_t* trans, const int32_t* count_cur,
                          const int32_t* key_rank, const int32_t* topk_next, const moe_predict_out& out,
                          const Workspace& ws, hipStream_t st);

// Replica slot map of a plan, and the row copies that move expert parameters
// into the slots and gradients back to the main ranks.
hipError_t launch_slot_map(const Dims& d, const moe_plan_out& plan, const moe_slot_out& out, int32_t* status,
                           hipStream_t st);
hipError_t launch_replica_pull(const Dims& d, const int32_t* slot_expert, const uint16_t* main_params, int64_t P,
                               uint16_t* replica_params, int32_t* status, hipStream_t st);
hipError_t launch_replica_push(const Dims& d, const int32_t* slot_expert, const uint16_t* replica_grads, int64_t P,
                               uint16_t* grad_accum, int32_t* status, hipStream_t st);

// LDS bytes the plan and scan kernels need for these dimensions.
size_t plan_lds_bytes(const Dims& d);
size_t scan_lds_bytes(const Dims& d);
size_t place_lds_bytes(const Dims& d);
size_t place_c16_elems(const Dims& d);
size_t dedup_scan_lds_bytes(const Dims& d);
// Workspace words of the pair kernel.
size_t pair_part_words(const Dims& d);

}  // namespace moe
