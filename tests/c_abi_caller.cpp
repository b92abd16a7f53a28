// A caller of the C ABI with no Python and no torch: device buffers from
// hipMalloc, a stream of its own.  Test helper for tests/test_gpu_c_caller.py.
//
//   c_abi_caller <dir>
// reads  <dir>/cfg.txt     "T E k R G H B" (the other fields: derived defaults)
//        <dir>/logits.f32  float [T][E]
//        <dir>/hidden.u16  bf16 bit patterns [T][H]
//        <dir>/omega.i32   int32 [R][E]  a routing matrix handed to the planner
//        <dir>/topk.i32    int32 [T][k]  the top-k that matrix counts
// and runs the path three ways on one handle:
//   step_*    moe_plan_step (one call)
//   staged_*  moe_plan_route, moe_plan_plan on the route's omega and topk_idx,
//             moe_plan_dispatch (three calls)
//   given_*   moe_plan_plan on omega.i32 / topk.i32, then moe_plan_dispatch
// writing <dir>/<way>_<name>.bin for every output (raw little-endian arrays,
// the layouts of include/moe_plan.h), then prints "ok".  Every output buffer
// is filled with 0xff bytes before each way, so each file holds what that
// way wrote.  Any failing call prints its name and code and exits non-zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "moe_plan.h"

namespace {

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(3);
  }
}

void abi_check(int rc, const char* what) {
  if (rc != MOE_OK) {
    std::fprintf(stderr, "%s returned %d\n", what, rc);
    std::exit(4);
  }
}

std::vector<char> read_file(const std::string& path, size_t bytes) {
  std::vector<char> buf(bytes);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(buf.data(), 1, bytes, f) != bytes) {
    std::fprintf(stderr, "cannot read %zu bytes of %s\n", bytes, path.c_str());
    std::exit(2);
  }
  std::fclose(f);
  return buf;
}

struct DevBuf {
  const char* name = nullptr;
  void* p = nullptr;
  size_t bytes = 0;
};

DevBuf alloc(const char* name, size_t bytes) {
  DevBuf b;
  b.name = name;
  b.bytes = bytes;
  hip_check(hipMalloc(&b.p, bytes > 0 ? bytes : 1), "hipMalloc");
  return b;
}

DevBuf upload(const std::string& path, size_t bytes) {
  DevBuf b = alloc("input", bytes);
  const std::vector<char> host = read_file(path, bytes);
  if (bytes > 0) hip_check(hipMemcpy(b.p, host.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy");
  return b;
}

void save(const std::string& dir, const std::string& way, const DevBuf& b) {
  std::vector<char> host(b.bytes);
  if (b.bytes > 0) hip_check(hipMemcpy(host.data(), b.p, b.bytes, hipMemcpyDeviceToHost), "hipMemcpy");
  const std::string path = dir + "/" + way + "_" + b.name + ".bin";
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(host.data(), 1, host.size(), f) != host.size()) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(2);
  }
  std::fclose(f);
}

template <typename T>
T* as(const DevBuf& b) {
  return static_cast<T*>(b.p);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 1;
  }
  const std::string dir = argv[1];
  moe_plan_config cfg{};
  {
    FILE* f = std::fopen((dir + "/cfg.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%d %d %d %d %d %d %d", &cfg.T, &cfg.E, &cfg.k, &cfg.R, &cfg.G, &cfg.H,
                          &cfg.replica_budget) != 7) {
      std::fprintf(stderr, "cannot read cfg.txt\n");
      return 2;
    }
    std::fclose(f);
  }
  cfg.slots_per_rank = 0;      // derived
  cfg.expert_bytes = -1;       // 9 H^2 / 4
  cfg.token_bytes = 0;         // 2 H
  cfg.max_refine_iters = 0;    // 4096

  moe_plan_sizes sz;
  abi_check(moe_plan_query(&cfg, &sz), "moe_plan_query");
  hip_check(hipSetDevice(0), "hipSetDevice");
  moe_plan_t h = nullptr;
  abi_check(moe_plan_create(&cfg, &h), "moe_plan_create");
  hipStream_t stream;
  hip_check(hipStreamCreate(&stream), "hipStreamCreate");

  const size_t i4 = sizeof(int32_t);
  DevBuf logits = upload(dir + "/logits.f32", (size_t)cfg.T * cfg.E * sizeof(float));
  DevBuf hidden = upload(dir + "/hidden.u16", (size_t)cfg.T * cfg.H * sizeof(uint16_t));
  DevBuf given_omega = upload(dir + "/omega.i32", (size_t)sz.omega * i4);
  DevBuf given_topk = upload(dir + "/topk.i32", (size_t)sz.topk * i4);

  std::vector<DevBuf> outs = {
      alloc("topk_idx", sz.topk * i4),        alloc("topk_val", sz.topk * sizeof(float)),
      alloc("count", sz.experts * i4),        alloc("omega", sz.omega * i4),
      alloc("cooc", sz.pair * i4),            alloc("n_inst", i4),
      alloc("inst_expert", sz.inst_cap * i4), alloc("inst_rank", sz.inst_cap * i4),
      alloc("inst_load", sz.inst_cap * i4),   alloc("rank_load", (size_t)cfg.R * i4),
      alloc("quota", sz.quota * i4),          alloc("slot_inst", sz.topk * i4),
      alloc("slot_rank", sz.topk * i4),       alloc("perm", sz.topk * i4),
      alloc("slot_pos", sz.topk * i4),        alloc("inst_offset", sz.inst_offset * i4),
      alloc("rank_offset", sz.rank_offset * i4), alloc("dispatch", sz.dispatch_elems * sizeof(uint16_t))};
  auto buf = [&](const char* name) -> const DevBuf& {
    for (const DevBuf& b : outs)
      if (std::string(b.name) == name) return b;
    std::fprintf(stderr, "no buffer %s\n", name);
    std::exit(2);
  };
  const moe_route_out route{as<int32_t>(buf("topk_idx")), as<float>(buf("topk_val")), as<int32_t>(buf("count")),
                            as<int32_t>(buf("omega")),    as<int32_t>(buf("cooc")),   nullptr};
  const moe_plan_out plan{as<int32_t>(buf("n_inst")),    as<int32_t>(buf("inst_expert")),
                          as<int32_t>(buf("inst_rank")), as<int32_t>(buf("inst_load")),
                          as<int32_t>(buf("rank_load")), as<int32_t>(buf("quota")),
                          as<int32_t>(buf("slot_inst")), as<int32_t>(buf("slot_rank"))};
  const moe_dispatch_out disp{as<int32_t>(buf("perm")), as<int32_t>(buf("slot_pos")), as<int32_t>(buf("inst_offset")),
                              as<int32_t>(buf("rank_offset")), as<uint16_t>(buf("dispatch"))};

  auto poison = [&]() {
    for (const DevBuf& b : outs) hip_check(hipMemsetAsync(b.p, 0xff, b.bytes, stream), "hipMemsetAsync");
  };
  auto finish = [&](const char* way) {
    hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
    int32_t flags = -1;
    abi_check(moe_plan_status(h, &flags), "moe_plan_status");
    if (flags != 0) {
      std::fprintf(stderr, "%s: status flags %d\n", way, flags);
      std::exit(5);
    }
    for (const DevBuf& b : outs) save(dir, way, b);
  };

  poison();
  abi_check(moe_plan_step(h, as<const float>(logits), nullptr, as<const uint16_t>(hidden), &route, &plan, &disp,
                          stream),
            "moe_plan_step");
  finish("step");

  poison();
  abi_check(moe_plan_route(h, as<const float>(logits), nullptr, &route, stream), "moe_plan_route");
  abi_check(moe_plan_plan(h, route.omega, route.topk_idx, &plan, stream), "moe_plan_plan");
  abi_check(moe_plan_dispatch(h, &plan, as<const uint16_t>(hidden), &disp, stream), "moe_plan_dispatch");
  finish("staged");

  poison();
  abi_check(moe_plan_plan(h, as<const int32_t>(given_omega), as<const int32_t>(given_topk), &plan, stream),
            "moe_plan_plan (given matrix)");
  abi_check(moe_plan_dispatch(h, &plan, as<const uint16_t>(hidden), &disp, stream), "moe_plan_dispatch");
  finish("given");

  moe_plan_destroy(h);
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  for (const DevBuf* b : {&logits, &hidden, &given_omega, &given_topk}) hip_check(hipFree(b->p), "hipFree");
  for (const DevBuf& b : outs) hip_check(hipFree(b.p), "hipFree");
  std::printf("ok\n");
  return 0;
}
