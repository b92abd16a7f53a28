// C ABI of the moe_plan library: validation, workspace ownership and the
// launch sequence of each call.  See include/moe_plan.h for the contract.
#include <new>

#include "internal.h"

struct moe_plan {
  moe::Dims d;
  moe_plan_config cfg;
  int device;
  moe::Workspace ws;
  void* ws_base;
  size_t ws_bytes;
  hipStream_t last_stream;  // stream of the last call that enqueued work (moe_plan_status waits for it)
  moe::KernelEvents gather_ev;  // moe_plan_set_events / moe_plan_set_gather_order: hooks around every gather launch
  bool acc_dirty;           // a step failed after its top-k was queued: the accumulator may hold counts
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kMaxLds = 160 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
  size_t status, tile_mask, tile_base, prev_mask, demand, einst_off, einst_list, rlist, colpre, pair_part, omega_acc;
  size_t place_aff, place_key, place_int, place_mem, place_c16, dd_mask, dd_cnt, dd_base, dd_count, pred_vote, total;
};

WsLayout ws_layout(const moe::Dims& d) {
  WsLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes > 0 ? bytes : 1); return at; };
  l.status = take(sizeof(int32_t));
  l.tile_mask = take(sizeof(uint64_t) * (size_t)d.NT * d.E);
  l.tile_base = take(sizeof(int32_t) * (size_t)d.NT * d.E);
  l.prev_mask = take(sizeof(uint64_t) * (size_t)d.NT * d.E);
  l.demand = take(sizeof(int32_t) * (size_t)d.M * d.E);
  l.einst_off = take(sizeof(int32_t) * (size_t)(d.E + 1));
  l.einst_list = take(sizeof(int32_t) * (size_t)d.cap);
  l.rlist = take(sizeof(int32_t) * (size_t)(d.E + 1));
  l.colpre = take(sizeof(int32_t) * (size_t)d.cap * d.R);
  l.pair_part = take(sizeof(int32_t) * moe::pair_part_words(d));
  l.omega_acc = take(sizeof(int32_t) * (size_t)d.R * d.E);
  l.place_aff = take(sizeof(int32_t) * (size_t)d.R * d.E);
  l.place_key = take(sizeof(uint64_t) * (size_t)d.R * d.R);
  l.place_int = take(sizeof(int32_t) * 4 * (size_t)d.E);
  l.place_mem = take(sizeof(int32_t) * (size_t)d.E);
  l.place_c16 = take(sizeof(uint16_t) * moe::place_c16_elems(d));
  l.dd_mask = take(sizeof(uint64_t) * (size_t)d.NT * d.R);
  l.dd_cnt = take(sizeof(int32_t) * (size_t)d.NT * d.R);
  l.dd_base = take(sizeof(int32_t) * (size_t)d.NT * d.R);
  l.dd_count = take(sizeof(int32_t) * (size_t)d.R);
  l.pred_vote = take(sizeof(double) * (size_t)d.E * d.R);
  l.total = o;
  return l;
}

}  // namespace

// Validates the configuration and derives every dimension the kernels use.
int moe::derive_dims(const moe_plan_config* c, moe::Dims* d) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->E < 1 || c->k < 1 || c->k > c->E || c->R < 1 || c->G < 1 || c->H < 1 ||
      c->replica_budget < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->R % c->G != 0 || c->T % c->R != 0 || c->E % c->R != 0) return MOE_ERR_INVALID_ARG;
  if (c->E > moe::kMaxE || c->k > moe::kMaxK || c->R > moe::kMaxR || c->G > moe::kMaxG ||
      c->replica_budget > moe::kMaxB)
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)c->T * c->k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  // The row copy launches up to four 256-thread workgroups per token, and a
  // dispatch holds fewer than 2^32 work-items.
  if (c->T >= 1 << 22) return MOE_ERR_UNSUPPORTED;
  if (c->token_bytes > ((int64_t)1 << 30) || c->expert_bytes > ((int64_t)1 << 62)) return MOE_ERR_UNSUPPORTED;
  moe::Dims x;
  x.T = c->T; x.E = c->E; x.k = c->k; x.R = c->R; x.G = c->G; x.H = c->H; x.B = c->replica_budget;
  x.M = c->R / c->G;
  x.Tr = c->T / c->R;
  x.Er = c->E / c->R;
  x.C = (x.Tr + moe::kTile - 1) / moe::kTile;
  x.NT = x.R * x.C;
  x.cap = x.E + x.B;
  const int per_dom = (x.B + x.M - 1) / x.M;
  x.n_slot = c->slots_per_rank > 0 ? c->slots_per_rank : (per_dom + x.G - 1) / x.G;
  if (x.n_slot > x.B) x.n_slot = x.B;  // more slots than replicas can never be used
  x.max_iters = c->max_refine_iters > 0 ? c->max_refine_iters : 4096;
  x.S = c->token_bytes > 0 ? c->token_bytes : 2LL * c->H;
  x.W = c->expert_bytes >= 0 ? c->expert_bytes : 9LL * c->H * c->H / 4;
  if (x.Er + x.n_slot > 1024) return MOE_ERR_UNSUPPORTED;
  if (moe::plan_lds_bytes(x) > kMaxLds || moe::scan_lds_bytes(x) > kMaxLds || moe::place_lds_bytes(x) > kMaxLds ||
      moe::dedup_scan_lds_bytes(x) > kMaxLds)
    return MOE_ERR_UNSUPPORTED;
  *d = x;
  return MOE_OK;
}

namespace {

// Makes `device` current for the duration of a call and gives the caller's
// current device back when the call returns.
class DeviceScope {
 public:
  explicit DeviceScope(int device) {
    if (hipGetDevice(&prev_) != hipSuccess) return;
    if (prev_ != device && hipSetDevice(device) != hipSuccess) return;
    switched_ = prev_ != device;
    ok_ = true;
  }
  ~DeviceScope() {
    if (switched_) (void)hipSetDevice(prev_);
  }
  DeviceScope(const DeviceScope&) = delete;
  DeviceScope& operator=(const DeviceScope&) = delete;
  bool ok() const { return ok_; }

 private:
  int prev_ = -1;
  bool switched_ = false;
  bool ok_ = false;
};

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" int moe_plan_query(const moe_plan_config* cfg, moe_plan_sizes* sz) {
  moe::Dims d;
  const int rc = moe::derive_dims(cfg, &d);
  if (rc != MOE_OK) return rc;
  if (!sz) return MOE_ERR_INVALID_ARG;
  sz->topk = (int64_t)d.T * d.k;
  sz->omega = (int64_t)d.R * d.E;
  sz->experts = d.E;
  sz->pair = (int64_t)d.E * d.E;
  sz->inst_cap = d.cap;
  sz->quota = (int64_t)d.R * d.cap;
  sz->inst_offset = d.cap + 1;
  sz->rank_offset = d.R + 1;
  sz->dispatch_elems = (int64_t)d.T * d.k * d.H;
  sz->n_slot = d.n_slot;
  sz->expert_bytes = d.W;
  sz->token_bytes = d.S;
  sz->max_refine_iters = d.max_iters;
  sz->workspace_bytes = (int64_t)ws_layout(d).total;
  return MOE_OK;
}

extern "C" int moe_plan_create(const moe_plan_config* cfg, moe_plan_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe::Dims d;
  const int rc = moe::derive_dims(cfg, &d);
  if (rc != MOE_OK) return rc;
  moe_plan* h = new (std::nothrow) moe_plan();
  if (!h) return MOE_ERR_INTERNAL;
  h->d = d;
  h->cfg = *cfg;
  h->last_stream = nullptr;
  h->gather_ev = moe::KernelEvents{nullptr, nullptr, nullptr, nullptr};
  h->acc_dirty = false;
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return MOE_ERR_HIP; }
  const WsLayout l = ws_layout(d);
  if (hipMalloc(&h->ws_base, l.total) != hipSuccess) { delete h; return MOE_ERR_HIP; }
  h->ws_bytes = l.total;
  char* b = static_cast<char*>(h->ws_base);
  h->ws.status = reinterpret_cast<int32_t*>(b + l.status);
  h->ws.tile_mask = reinterpret_cast<uint64_t*>(b + l.tile_mask);
  h->ws.tile_base = reinterpret_cast<int32_t*>(b + l.tile_base);
  h->ws.prev_mask = reinterpret_cast<uint64_t*>(b + l.prev_mask);
  h->ws.demand = reinterpret_cast<int32_t*>(b + l.demand);
  h->ws.einst_off = reinterpret_cast<int32_t*>(b + l.einst_off);
  h->ws.einst_list = reinterpret_cast<int32_t*>(b + l.einst_list);
  h->ws.rlist = reinterpret_cast<int32_t*>(b + l.rlist);
  h->ws.colpre = reinterpret_cast<int32_t*>(b + l.colpre);
  h->ws.pair_part = reinterpret_cast<int32_t*>(b + l.pair_part);
  h->ws.omega_acc = reinterpret_cast<int32_t*>(b + l.omega_acc);
  h->ws.place_aff = reinterpret_cast<int32_t*>(b + l.place_aff);
  h->ws.place_key = reinterpret_cast<uint64_t*>(b + l.place_key);
  h->ws.place_int = reinterpret_cast<int32_t*>(b + l.place_int);
  h->ws.place_mem = reinterpret_cast<int32_t*>(b + l.place_mem);
  h->ws.place_c16 = reinterpret_cast<uint16_t*>(b + l.place_c16);
  h->ws.dd_mask = reinterpret_cast<uint64_t*>(b + l.dd_mask);
  h->ws.dd_cnt = reinterpret_cast<int32_t*>(b + l.dd_cnt);
  h->ws.dd_base = reinterpret_cast<int32_t*>(b + l.dd_base);
  h->ws.dd_count = reinterpret_cast<int32_t*>(b + l.dd_count);
  h->ws.pred_vote = reinterpret_cast<double*>(b + l.pred_vote);
  if (hipMemset(h->ws_base, 0, l.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(h->ws_base);
    delete h;
    return MOE_ERR_HIP;
  }
  *out = h;
  return MOE_OK;
}

int moe::check_step_args(const moe::Dims& d, const float* logits, const uint16_t* hidden, const moe_route_out* route,
                         const moe_plan_out* plan, const moe_dispatch_out* out);

namespace {

int check_route_out(const moe::Dims& d, const moe_route_out* out) {
  if (!out || !out->expert_count || !out->omega) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && !out->topk_idx) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_plan_out(const moe::Dims& d, const moe_plan_out* out) {
  if (!out || !out->n_inst || !out->inst_expert || !out->inst_rank || !out->inst_load || !out->rank_load ||
      !out->quota)
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!out->slot_inst || !out->slot_rank)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_dispatch_out(const moe::Dims& d, const moe_dispatch_out* out) {
  if (!out || !out->inst_offset || !out->rank_offset) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!out->perm || !out->slot_pos || !out->dispatch)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

int moe::check_step_args(const moe::Dims& d, const float* logits, const uint16_t* hidden, const moe_route_out* route,
                         const moe_plan_out* plan, const moe_dispatch_out* out) {
  if (check_route_out(d, route) != MOE_OK || check_plan_out(d, plan) != MOE_OK || check_dispatch_out(d, out) != MOE_OK)
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!logits || !hidden)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

namespace {

// Set-up shared by the calls that enqueue work: clears an error an earlier
// HIP call of the caller left behind (so that a failure reported by this
// call is its own) and remembers the stream for moe_plan_status.
hipStream_t begin_call(moe_plan_t h, void* stream) {
  (void)hipGetLastError();
  h->last_stream = static_cast<hipStream_t>(stream);
  return h->last_stream;
}

}  // namespace

extern "C" int moe_plan_route(moe_plan_t h, const float* logits, const int32_t* prev_topk, const moe_route_out* out,
                              void* stream) {
  if (!h || check_route_out(h->d, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  if (d.T > 0 && !logits) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  const int32_t* prev = (prev_topk && out->trans) ? prev_topk : nullptr;
  // The presence masks live in the workspace; the scan reads them for the
  // routing matrix and counts (no tile prefix is needed here) and the pair
  // counts run beside it in the same launch.
  hipError_t e = moe::launch_route_topk(d, logits, prev, out->topk_idx, out->topk_val, h->ws.tile_mask,
                                        h->ws.prev_mask, nullptr, h->ws.status, st);
  if (e == hipSuccess)
    e = moe::launch_scan_pairs(d, h->ws.tile_mask, nullptr, out->omega, out->expert_count, h->ws.prev_mask,
                               out->cooc, prev ? out->trans : nullptr, h->ws.pair_part, st);
  return hip_rc(e);
}

extern "C" int moe_plan_hist(moe_plan_t h, const int32_t* topk_idx, const int32_t* prev_topk, const moe_route_out* out,
                             void* stream) {
  if (!h || !out || !out->expert_count || !out->omega) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  if (d.T > 0 && !topk_idx) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  const int32_t* prev = (prev_topk && out->trans) ? prev_topk : nullptr;
  hipError_t e = moe::launch_build_masks(d, topk_idx, prev, h->ws.tile_mask, h->ws.prev_mask, h->ws.status, st);
  if (e == hipSuccess)
    e = moe::launch_scan_pairs(d, h->ws.tile_mask, nullptr, out->omega, out->expert_count, h->ws.prev_mask,
                               out->cooc, prev ? out->trans : nullptr, h->ws.pair_part, st);
  return hip_rc(e);
}

extern "C" int moe_plan_plan(moe_plan_t h, const int32_t* omega, const int32_t* topk_idx, const moe_plan_out* out,
                             void* stream) {
  if (!h || !omega || check_plan_out(h->d, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  if (d.T > 0 && !topk_idx) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  // The presence masks of the given top-k (checking every row), then the
  // solver on the given routing matrix while extra workgroups of its launch
  // build the tile prefix and compare the matrix with the masks' own, then
  // the quotas, then each slot's instance and rank.
  hipError_t e = moe::launch_build_masks(d, topk_idx, nullptr, h->ws.tile_mask, nullptr, h->ws.status, st);
  const moe::ScanJob scan{d.T > 0 ? h->ws.tile_mask : nullptr, h->ws.tile_base, nullptr, nullptr, omega};
  if (e == hipSuccess)
    e = moe::launch_plan(d, omega, scan, nullptr, nullptr, nullptr, nullptr, *out, nullptr, nullptr, h->ws,
                         moe::pipelined(h->gather_ev), st);
  if (e == hipSuccess)
    e = moe::launch_assign(d, topk_idx, h->ws.tile_mask, h->ws.tile_base, *out, h->ws, nullptr, 0, st);
  return hip_rc(e);
}

extern "C" int moe_plan_dispatch(moe_plan_t h, const moe_plan_out* plan, const uint16_t* hidden,
                                 const moe_dispatch_out* out, void* stream) {
  if (!h || !plan || check_dispatch_out(h->d, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  if (!plan->n_inst || !plan->inst_rank || !plan->inst_load) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  if (d.T > 0 && (!plan->slot_inst || !plan->slot_rank || !hidden)) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  return hip_rc(moe::launch_gather(d, *plan, hidden, out->perm, out->slot_pos, out->inst_offset, out->rank_offset,
                                   out->dispatch, h->ws, h->gather_ev, st));
}

extern "C" int moe_plan_step(moe_plan_t h, const float* logits, const int32_t* prev_topk, const uint16_t* hidden,
                             const moe_route_out* route, const moe_plan_out* plan, const moe_dispatch_out* out,
                             void* stream) {
  if (!h || moe::check_step_args(h->d, logits, hidden, route, plan, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  // If a launch fails after the top-k was queued, the accumulator may keep
  // counts; the next call then clears it first.
  const int64_t re = (int64_t)d.R * d.E;
  hipError_t e = hipSuccess;
  if (h->acc_dirty) {
    e = moe::launch_zero(h->ws.omega_acc, re, st);
    if (e != hipSuccess) return hip_rc(e);
    h->acc_dirty = false;
  }
  h->acc_dirty = true;  // until the launch that clears the accumulator is queued
  e = moe::enqueue_step(d, h->ws, logits, prev_topk, hidden, *route, *plan, *out, h->gather_ev, st);
  if (e == hipSuccess) h->acc_dirty = false;
  return hip_rc(e);
}

hipError_t moe::enqueue_step(const moe::Dims& d, const moe::Workspace& ws, const float* logits,
                             const int32_t* prev_topk, const uint16_t* hidden, const moe_route_out& route,
                             const moe_plan_out& plan, const moe_dispatch_out& out, const moe::KernelEvents& ev,
                             hipStream_t st) {
  const int32_t* prev = (prev_topk && route.trans) ? prev_topk : nullptr;
  // On `st`: top-k (which also accumulates the routing matrix into the
  // workspace accumulator, zero on entry) -> plan (the solver reads the
  // accumulator; workgroups on the CUs it leaves idle write the tile prefix,
  // the routing matrix and counts outputs and the pair-count partials) ->
  // quotas and dispatch offsets (read the accumulator too; extra workgroups
  // sum the pair-count partials) -> slot instances + gather, which zero the
  // accumulator again: the handle carries no state from one call to the
  // next, so the call can be captured in a HIP graph and replayed.
  const int64_t re = (int64_t)d.R * d.E;
  int32_t* acc = ws.omega_acc;
  hipError_t e = moe::launch_route_topk(d, logits, prev, route.topk_idx, route.topk_val, ws.tile_mask, ws.prev_mask,
                                        acc, ws.status, st);
  const moe::ScanJob scan{ws.tile_mask, ws.tile_base, route.omega, route.expert_count, nullptr};
  int32_t* trans = prev ? route.trans : nullptr;
  if (e == hipSuccess)
    e = moe::launch_plan(d, acc, scan, ws.prev_mask, route.cooc, trans, ws.pair_part, plan, out.inst_offset,
                         out.rank_offset, ws, moe::pipelined(ev), st);
  if (moe::gather_can_assign(d, hidden, out.dispatch) && moe::copy_in_one_part(d)) {
    // the gather assigns its token's slots itself, overlapping the row load
    if (e == hipSuccess)
      e = moe::launch_assign_gather(d, route.topk_idx, ws.tile_mask, ws.tile_base, plan, out.inst_offset, hidden,
                                    out.perm, out.slot_pos, out.dispatch, ws, acc, re, ev, st);
  } else {
    // a copy in several parts per token: the slots first (before the copy's
    // ordering hooks, so beside another batch's copy), then the parts
    if (e == hipSuccess) e = moe::launch_assign(d, route.topk_idx, ws.tile_mask, ws.tile_base, plan, ws, acc, re, st);
    if (e == hipSuccess)
      e = moe::launch_gather_rows(d, plan, hidden, out.perm, out.slot_pos, out.inst_offset, out.dispatch, ws, ev, st);
  }
  return e;
}

extern "C" int moe_plan_combine(moe_plan_t h, const float* topk_val, const int32_t* slot_pos,
                                const uint16_t* expert_out, uint16_t* out, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  const moe::Dims& d = h->d;
  if (d.T > 0 && (!topk_val || !slot_pos || !expert_out || !out)) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  hipStream_t st = begin_call(h, stream);
  return hip_rc(moe::launch_combine(d, topk_val, slot_pos, expert_out, out, h->ws.status, st));
}

extern "C" int moe_plan_place(moe_plan_t h, const int32_t* cooc, int32_t max_swaps, const moe_place_out* out,
                              void* stream) {
  if (!h || !cooc || !out || !out->expert_rank || !out->rank_experts || !out->intra || !out->n_swaps)
    return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_place(h->d, cooc, max_swaps, *out, h->ws, begin_call(h, stream)));
}

namespace {

int check_dedup(const moe::Dims& d, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                const moe_dedup_out* out) {
  if (!out || !out->rank_rows) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!slot_key || !out->tok_ranks)) return MOE_ERR_INVALID_ARG;
  if (key_rank && n_keys < 1) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_plan_dedup_count(moe_plan_t h, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                                    const moe_dedup_out* out, void* stream) {
  if (!h || check_dedup(h->d, slot_key, key_rank, n_keys, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(
      moe::launch_dedup(h->d, slot_key, key_rank, n_keys, nullptr, *out, h->ws, begin_call(h, stream)));
}

extern "C" int moe_plan_dedup_dispatch(moe_plan_t h, const int32_t* slot_key, const int32_t* key_rank,
                                       int32_t n_keys, const uint16_t* hidden, const moe_dedup_out* out,
                                       void* stream) {
  if (!h || check_dedup(h->d, slot_key, key_rank, n_keys, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  if (!out->n_rows || !out->rank_row_offset) return MOE_ERR_INVALID_ARG;
  if (h->d.T > 0 && (!hidden || !out->row_token || !out->row_slots || !out->slot_row || !out->ddispatch))
    return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  // a non-null row source selects the layout and copy; T = 0 still writes the offsets
  static const uint16_t kNoRows = 0;
  const uint16_t* src = hidden ? hidden : &kNoRows;
  return hip_rc(
      moe::launch_dedup(h->d, slot_key, key_rank, n_keys, src, *out, h->ws, begin_call(h, stream)));
}

extern "C" int moe_plan_quality(moe_plan_t h, const moe_plan_out* plan, int64_t* out, void* stream) {
  if (!h || !plan || !out || !plan->n_inst || !plan->inst_expert || !plan->inst_rank || !plan->rank_load ||
      !plan->quota)
    return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_quality(h->d, *plan, out, h->ws.status, begin_call(h, stream)));
}

extern "C" int moe_plan_predict(moe_plan_t h, const int32_t* topk_cur, const int32_t* trans, const int32_t* count_cur,
                                const int32_t* key_rank, const int32_t* topk_next, const moe_predict_out* out,
                                void* stream) {
  if (!h || !trans || !count_cur || !out || !out->rank_tokens) return MOE_ERR_INVALID_ARG;
  if (h->d.T > 0 && (!topk_cur || !out->pred)) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_predict(h->d, topk_cur, trans, count_cur, key_rank, topk_next, *out, h->ws,
                                    begin_call(h, stream)));
}

extern "C" int moe_plan_slot_map(moe_plan_t h, const moe_plan_out* plan, const moe_slot_out* out, void* stream) {
  if (!h || !plan || !out || !plan->n_inst || !plan->inst_expert || !plan->inst_rank || !out->inst_slot)
    return MOE_ERR_INVALID_ARG;
  if (h->d.n_slot > 0 && (!out->slot_expert || !out->slot_main)) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_slot_map(h->d, *plan, *out, h->ws.status, begin_call(h, stream)));
}

extern "C" int moe_plan_replica_pull(moe_plan_t h, const int32_t* slot_expert, const uint16_t* main_params,
                                     int64_t param_elems, uint16_t* replica_params, void* stream) {
  if (!h || param_elems < 0) return MOE_ERR_INVALID_ARG;
  if (h->d.n_slot > 0 && param_elems > 0 && (!slot_expert || !main_params || !replica_params))
    return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_replica_pull(h->d, slot_expert, main_params, param_elems, replica_params, h->ws.status,
                                         begin_call(h, stream)));
}

extern "C" int moe_plan_replica_push(moe_plan_t h, const int32_t* slot_expert, const uint16_t* replica_grads,
                                     int64_t param_elems, uint16_t* grad_accum, void* stream) {
  if (!h || param_elems < 0) return MOE_ERR_INVALID_ARG;
  if (h->d.n_slot > 0 && param_elems > 0 && (!slot_expert || !replica_grads || !grad_accum))
    return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  return hip_rc(moe::launch_replica_push(h->d, slot_expert, replica_grads, param_elems, grad_accum, h->ws.status,
                                         begin_call(h, stream)));
}

extern "C" int moe_plan_set_events(moe_plan_t h, void* gather_begin, void* gather_end) {
  if (!h || (gather_begin == nullptr) != (gather_end == nullptr)) return MOE_ERR_INVALID_ARG;
  h->gather_ev.begin = static_cast<hipEvent_t>(gather_begin);
  h->gather_ev.end = static_cast<hipEvent_t>(gather_end);
  return MOE_OK;
}

extern "C" int moe_plan_set_gather_order(moe_plan_t h, void* wait_event, void* done_event) {
  if (!h) return MOE_ERR_INVALID_ARG;
  h->gather_ev.wait = static_cast<hipEvent_t>(wait_event);
  h->gather_ev.done = static_cast<hipEvent_t>(done_event);
  return MOE_OK;
}

extern "C" int moe_plan_device_info(int device, int64_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  const hipDeviceAttribute_t attrs[5] = {hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeClockRate,
                                         hipDeviceAttributeMemoryClockRate, hipDeviceAttributeMemoryBusWidth,
                                         hipDeviceAttributeL2CacheSize};
  for (int i = 0; i < 5; ++i) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, attrs[i], device) != hipSuccess) return MOE_ERR_HIP;
    out[i] = v;
  }
  size_t free_b = 0, total_b = 0;
  const DeviceScope on_device(device);
  if (!on_device.ok() || hipMemGetInfo(&free_b, &total_b) != hipSuccess) return MOE_ERR_HIP;
  out[5] = (int64_t)total_b;
  return MOE_OK;
}

extern "C" int moe_plan_status(moe_plan_t h, int32_t* host_flags) {
  if (!h || !host_flags) return MOE_ERR_INVALID_ARG;
  const DeviceScope on_device(h->device);
  if (!on_device.ok()) return MOE_ERR_HIP;
  // In order on the last call's stream: read the word, clear it, then wait
  // for that stream alone (other streams keep running).
  hipStream_t st = h->last_stream;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, h->ws.status, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_zero(h->ws.status, 1, st) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
  *host_flags = v;
  return MOE_OK;
}

extern "C" void moe_plan_destroy(moe_plan_t h) {
  if (!h) return;
  const DeviceScope on_device(h->device);
  if (on_device.ok()) {
    (void)hipDeviceSynchronize();
    (void)hipFree(h->ws_base);
  }
  delete h;
}
