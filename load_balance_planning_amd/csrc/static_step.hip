// moe_plan_step_static: the single-call step for callers that cannot call
// hipMalloc (work under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  It runs exactly the launches of moe_plan_step, with
// the workspace carved out of a fixed device array instead of a handle.
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy (kStaticScratchBytes) until the process ends.  Host
// code never uses the array's name as an address -- on the host it is only a
// stand-in for the symbol -- but the device address hipGetSymbolAddress
// returns, looked up once per device with that device current.
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's copy of the array (the current device).
hipError_t scratch_address(int device, void** out) {
  std::call_once(g_scratch_once[device], [device]() {
    g_scratch_err[device] = hipGetSymbolAddress(&g_scratch_ptr[device], HIP_SYMBOL(scratch));
  });
  *out = g_scratch_ptr[device];
  return g_scratch_err[device];
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The parts of the handle workspace that the step uses, laid out from offset
// 0 of the array; returns the bytes needed.  The status word is the caller's.
size_t step_layout(const moe::Dims& d, bool with_prev, char* base, moe::Workspace* ws) {
  size_t o = 0;
  auto take = [&](size_t bytes) -> char* {
    char* at = base ? base + o : nullptr;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  moe::Workspace w{};
  w.tile_mask = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)d.NT * d.E));
  w.tile_base = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)d.NT * d.E));
  w.prev_mask = with_prev ? reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)d.NT * d.E)) : nullptr;
  w.demand = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)d.M * d.E));
  w.einst_off = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)(d.E + 1)));
  w.einst_list = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)d.cap));
  w.rlist = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)(d.E + 1)));
  w.colpre = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)d.cap * d.R));
  w.pair_part = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * moe::pair_part_words(d)));
  w.omega_acc = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)d.R * d.E));
  if (ws) *ws = w;
  return o;
}

}  // namespace

extern "C" int moe_plan_step_static(const moe_plan_config* cfg, const float* logits, const int32_t* prev_topk,
                                    const uint16_t* hidden, const moe_route_out* route, const moe_plan_out* plan,
                                    const moe_dispatch_out* out, int32_t* status, void* stream) {
  moe::Dims d;
  int rc = moe::derive_dims(cfg, &d);
  if (rc != MOE_OK) return rc;
  if (!status || moe::check_step_args(d, logits, hidden, route, plan, out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  const bool with_prev = prev_topk && route->trans;
  if (step_layout(d, with_prev, nullptr, nullptr) > kStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // a failure reported below is this call's own
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return MOE_ERR_HIP;
  if (device < 0 || device >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* base = nullptr;
  if (scratch_address(device, &base) != hipSuccess || !base) return MOE_ERR_HIP;
  moe::Workspace ws;
  step_layout(d, with_prev, static_cast<char*>(base), &ws);
  ws.status = status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The array keeps whatever the last call on this device left: the status
  // word and the routing-matrix accumulator start at zero (fill kernels, which
  // a graph capture records as ordinary kernels); every other part is written
  // before it is read.
  hipError_t e = moe::launch_zero(status, 1, st);
  if (e == hipSuccess) e = moe::launch_zero(ws.omega_acc, (int64_t)d.R * d.E, st);
  if (e == hipSuccess)
    e = moe::enqueue_step(d, ws, logits, with_prev ? prev_topk : nullptr, hidden, *route, *plan, *out,
                          moe::KernelEvents{nullptr, nullptr, nullptr, nullptr}, st);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
