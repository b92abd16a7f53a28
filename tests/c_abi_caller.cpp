// A caller of the C ABI with no Python and no torch: device buffers from
// hipMalloc, a stream of its own, the whole pass in one moe_plan_step call.
// Test helper for tests/test_gpu_c_caller.py.
//
//   c_abi_caller <dir>
// reads  <dir>/cfg.txt     "T E k R G H B" (the other fields: derived defaults)
//        <dir>/logits.f32  float [T][E]
//        <dir>/hidden.u16  bf16 bit patterns [T][H]
// writes <dir>/<name>.bin for every output of the step (raw little-endian
// arrays, the layouts of include/moe_plan.h) and prints "ok".  Any failing
// call prints its name and code and exits non-zero.
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
  void* p = nullptr;
  size_t bytes = 0;
};

DevBuf alloc(size_t bytes) {
  DevBuf b;
  b.bytes = bytes;
  hip_check(hipMalloc(&b.p, bytes > 0 ? bytes : 1), "hipMalloc");
  return b;
}

void save(const std::string& dir, const char* name, const DevBuf& b) {
  std::vector<char> host(b.bytes);
  if (b.bytes > 0) hip_check(hipMemcpy(host.data(), b.p, b.bytes, hipMemcpyDeviceToHost), "hipMemcpy");
  const std::string path = dir + "/" + name + ".bin";
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(host.data(), 1, host.size(), f) != host.size()) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(2);
  }
  std::fclose(f);
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
  const size_t logits_bytes = (size_t)cfg.T * cfg.E * sizeof(float);
  const size_t hidden_bytes = (size_t)cfg.T * cfg.H * sizeof(uint16_t);
  DevBuf logits = alloc(logits_bytes), hidden = alloc(hidden_bytes);
  {
    const std::vector<char> lg = read_file(dir + "/logits.f32", logits_bytes);
    const std::vector<char> hd = read_file(dir + "/hidden.u16", hidden_bytes);
    hip_check(hipMemcpy(logits.p, lg.data(), logits_bytes, hipMemcpyHostToDevice), "hipMemcpy");
    hip_check(hipMemcpy(hidden.p, hd.data(), hidden_bytes, hipMemcpyHostToDevice), "hipMemcpy");
  }
  DevBuf topk_idx = alloc(sz.topk * i4), topk_val = alloc(sz.topk * sizeof(float)), count = alloc(sz.experts * i4);
  DevBuf omega = alloc(sz.omega * i4), cooc = alloc(sz.pair * i4);
  DevBuf tile_mask = alloc(sz.tile_words * sizeof(uint64_t)), tile_base = alloc(sz.tile_words * i4);
  DevBuf n_inst = alloc(i4), inst_expert = alloc(sz.inst_cap * i4), inst_rank = alloc(sz.inst_cap * i4);
  DevBuf inst_load = alloc(sz.inst_cap * i4), rank_load = alloc((size_t)cfg.R * i4), quota = alloc(sz.quota * i4);
  DevBuf slot_inst = alloc(sz.topk * i4), slot_rank = alloc(sz.topk * i4);
  DevBuf inst_offset = alloc(sz.inst_offset * i4), rank_offset = alloc(sz.rank_offset * i4);
  DevBuf perm = alloc(sz.topk * i4), slot_pos = alloc(sz.topk * i4);
  DevBuf dispatch = alloc(sz.dispatch_elems * sizeof(uint16_t));

  moe_route_out route{static_cast<int32_t*>(topk_idx.p), static_cast<float*>(topk_val.p),
                      static_cast<int32_t*>(count.p),    static_cast<int32_t*>(omega.p),
                      static_cast<int32_t*>(cooc.p),     nullptr,
                      static_cast<uint64_t*>(tile_mask.p), static_cast<int32_t*>(tile_base.p)};
  moe_plan_out plan{static_cast<int32_t*>(n_inst.p),    static_cast<int32_t*>(inst_expert.p),
                    static_cast<int32_t*>(inst_rank.p), static_cast<int32_t*>(inst_load.p),
                    static_cast<int32_t*>(rank_load.p), static_cast<int32_t*>(quota.p),
                    static_cast<int32_t*>(slot_inst.p), static_cast<int32_t*>(slot_rank.p),
                    static_cast<int32_t*>(inst_offset.p), static_cast<int32_t*>(rank_offset.p)};
  moe_dispatch_out disp{static_cast<int32_t*>(perm.p), static_cast<int32_t*>(slot_pos.p),
                        static_cast<uint16_t*>(dispatch.p)};

  abi_check(moe_plan_step(h, static_cast<const float*>(logits.p), nullptr, static_cast<const uint16_t*>(hidden.p),
                          &route, &plan, &disp, stream),
            "moe_plan_step");
  hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
  int32_t flags = -1;
  abi_check(moe_plan_status(h, &flags), "moe_plan_status");
  if (flags != 0) {
    std::fprintf(stderr, "status flags %d\n", flags);
    return 5;
  }
  const struct {
    const char* name;
    const DevBuf* buf;
  } outs[] = {{"topk_idx", &topk_idx}, {"topk_val", &topk_val}, {"count", &count},     {"omega", &omega},
              {"cooc", &cooc},         {"n_inst", &n_inst},     {"inst_expert", &inst_expert},
              {"inst_rank", &inst_rank}, {"inst_load", &inst_load}, {"rank_load", &rank_load},
              {"quota", &quota},       {"slot_inst", &slot_inst}, {"slot_rank", &slot_rank},
              {"inst_offset", &inst_offset}, {"rank_offset", &rank_offset}, {"perm", &perm},
              {"slot_pos", &slot_pos}, {"dispatch", &dispatch}};
  for (const auto& o : outs) save(dir, o.name, *o.buf);

  moe_plan_destroy(h);
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  for (const DevBuf* b : {&logits, &hidden, &topk_idx, &topk_val, &count, &omega, &cooc, &tile_mask, &tile_base,
                          &n_inst, &inst_expert, &inst_rank, &inst_load, &rank_load, &quota, &slot_inst,
                          &slot_rank, &inst_offset, &rank_offset, &perm, &slot_pos, &dispatch})
    hip_check(hipFree(b->p), "hipFree");
  std::printf("ok\n");
  return 0;
}
