// Host-only check of the planner and the C-ABI validation layer, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py compiles it with g++ together
// with csrc/plan.cpp and csrc/mla_api.cpp).  No kernel is compiled in: the launchers below
// abort if reached, and nothing here may reach them (every call either fails validation or
// only plans).  Prints "ok" and returns 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla.h"
#include "mla_internal.h"

namespace mla {
[[noreturn]] static void no_kernels(const char* what) {
  std::fprintf(stderr, "host check reached a kernel launcher: %s\n", what);
  std::abort();
}
int launch_decode(const DecodeArgs&, int, bool, int, void*, bool) { no_kernels("decode"); }
int launch_merge(const MergeArgs&, bool, void*) { no_kernels("merge"); }
int launch_merge_dev(const MergeArgs&, bool, void*) { no_kernels("merge_dev"); }
int launch_fill_zero(void*, size_t, void*) { no_kernels("fill_zero"); }
int launch_gather(const void*, const int32_t*, void*, int32_t, int32_t, int64_t, int32_t, int32_t, int32_t, int32_t,
                  void*) {
  no_kernels("gather");
}
int launch_q_absorb(const LayerArgs&, void*) { no_kernels("q_absorb"); }
int launch_kv_append(const LayerArgs&, void*) { no_kernels("kv_append"); }
int launch_out_absorb(const LayerArgs&, bool, bool, void*) { no_kernels("out_absorb"); }
const char* hip_error_string(int) { return "no kernels in the host check"; }
int noalloc_scratch(void**) { no_kernels("noalloc_scratch"); }
int launch_stream_probe(const void*, int64_t, int, void*) { no_kernels("stream_probe"); }
}  // namespace mla

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::printf("check failed at line %d: %s (%s)\n", __LINE__, #c, mla_last_error()); \
      return false;                                                           \
    }                                                                         \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {   // xorshift64*, uniform enough for a fuzz
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return (uint32_t)((g_rng * 2685821657736338717ull) >> 33) % n;
}

// One random problem: plan it and check the schedule's invariants.
static bool fuzz_one(int iter) {
  static const int pages[] = {16, 32, 48, 64, 80, 1024};
  static const int rows[] = {16, 32, 48, 64, 128, 256};
  mla_problem_t p;
  std::memset(&p, 0, sizeof p);
  p.batch = 1 + (int)rnd(iter % 7 == 0 ? 1200 : 70);
  const int R = rows[rnd(6)];
  p.q_len = (R == 256 || rnd(3) == 0) && R % 32 == 0 ? 2 : 1;
  p.num_heads = R / p.q_len;
  p.head_dim_qk = 576;
  p.head_dim_v = 512;
  p.page_size = pages[rnd(6)];
  p.out_dtype = rnd(2) ? MLA_DTYPE_FP32 : MLA_DTYPE_BF16;
  p.causal = (int32_t)rnd(2);
  p.kv_dtype = rnd(3) == 0 ? MLA_KV_FP8_E4M3 : MLA_KV_BF16;
  const int max_len = iter % 11 == 0 ? (1 << 20) : iter % 3 == 0 ? 70000 : 3000;
  std::vector<int32_t> lens(p.batch);
  int64_t pages_used = 0;
  int32_t maxp = 1;
  for (auto& L : lens) {
    const uint32_t k = rnd(10);
    L = k == 0 ? 0 : k == 1 ? (int32_t)rnd(17) : (int32_t)rnd((uint32_t)max_len + 1);
    if (p.batch > 200) L = (int32_t)rnd(300);
    const int32_t np_ = (L + p.page_size - 1) / p.page_size;
    pages_used += np_;
    if (np_ > maxp) maxp = np_;
  }
  p.max_pages_per_seq = maxp + (int32_t)rnd(3);
  p.num_pages = (int32_t)pages_used + 1;
  mla_plan_options_t opt;
  std::memset(&opt, 0, sizeof opt);
  opt.num_cus = 1 + (int32_t)rnd(rnd(4) == 0 ? 16 : 1024);
  opt.force_splits = rnd(6) == 0 ? 1 + (int32_t)rnd(1000) : 0;
  const int rpg_opts[] = {0, 16, 32, 64, 128};
  opt.rows_per_group = rpg_opts[rnd(5)];
  const bool rpg_ok = opt.rows_per_group <= 16 ||
                      (R % opt.rows_per_group == 0 && (opt.rows_per_group != 32 || p.kv_dtype == MLA_KV_BF16));
  mla_plan_t plan = nullptr;
  const mla_status_t st = mla_plan(&p, lens.data(), &opt, &plan);
  if (!rpg_ok) {
    CHECK(st == MLA_ERR_UNSUPPORTED && plan == nullptr);
    return true;
  }
  CHECK(st == MLA_OK && plan != nullptr);
  mla_plan_info_t info;
  CHECK(mla_plan_get_info(plan, &info) == MLA_OK);
  CHECK(info.row_groups * info.rows_per_group == R);
  CHECK(info.metadata_bytes > 0 && info.metadata_bytes <= info.workspace_bytes && info.workspace_bytes % 256 == 0);
  CHECK((size_t)info.workspace_bytes == mla_plan_workspace_bytes(plan));
  CHECK((int64_t)info.workspace_bytes >=
        info.metadata_bytes + (int64_t)info.num_partials * R * 4 * (1 + 512));
  std::vector<int32_t> seg(4 * (size_t)(info.num_segments > 0 ? info.num_segments : 1));
  std::vector<int32_t> off((size_t)info.num_workers + 1);
  CHECK(mla_plan_get_segments(plan, seg.data(), (int64_t)seg.size(), off.data(), (int64_t)off.size()) == MLA_OK);
  CHECK(off[0] == 0 && off[info.num_workers] == info.num_segments);
  if (opt.force_splits == 0) CHECK(info.num_workers <= opt.num_cus);
  std::vector<int64_t> covered(p.batch, 0);
  std::vector<int32_t> pieces_of(p.batch, 0), slot_next(p.batch, -2);
  int64_t partials = 0;
  for (int w = 0; w < info.num_workers; ++w) {
    CHECK(off[w] <= off[w + 1]);
    for (int i = off[w]; i < off[w + 1]; ++i) {
      const int32_t b = seg[4 * i], t0 = seg[4 * i + 1], t1 = seg[4 * i + 2], slot = seg[4 * i + 3];
      CHECK(b >= 0 && b < p.batch);
      CHECK(t0 == covered[b] && t1 >= t0 && t1 <= lens[b] && t0 % 16 == 0);
      covered[b] = t1;
      if (slot >= 0) {
        CHECK(slot < info.num_partials);
        CHECK(slot_next[b] == -2 || slot == slot_next[b]);
        slot_next[b] = slot + 1;
        ++partials;
      }
      ++pieces_of[b];
    }
  }
  for (int b = 0; b < p.batch; ++b) {
    CHECK(covered[b] == lens[b]);
    CHECK((pieces_of[b] == 1) == (slot_next[b] == -2));
  }
  CHECK(partials == info.num_partials);
  // a too-small capacity is refused without writing past it
  if (info.num_segments > 0) {
    std::vector<int32_t> small(4 * (size_t)info.num_segments - 1);
    CHECK(mla_plan_get_segments(plan, small.data(), (int64_t)small.size(), nullptr, 0) == MLA_ERR_INVALID_ARGUMENT);
  }
  mla_plan_destroy(plan);
  return true;
}

static bool validation_paths() {
  mla_problem_t p;
  std::memset(&p, 0, sizeof p);
  p.batch = 2;
  p.q_len = 1;
  p.num_heads = 16;
  p.head_dim_qk = 576;
  p.head_dim_v = 512;
  p.page_size = 64;
  p.num_pages = 4;
  p.max_pages_per_seq = 2;
  int32_t lens[2] = {100, 50};
  mla_plan_options_t opt;
  std::memset(&opt, 0, sizeof opt);
  opt.num_cus = 256;
  mla_plan_t plan = nullptr;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_OK);
  const size_t n = mla_plan_workspace_bytes(plan);
  char* fake = (char*)(uintptr_t)(1 << 20);   // never dereferenced: every call below is refused
  CHECK(mla_plan_upload(plan, nullptr, n, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_plan_upload(plan, fake + 16, n, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_plan_upload(plan, fake, n - 1, nullptr) == MLA_ERR_WORKSPACE_TOO_SMALL);
  CHECK(mla_decode(plan, fake, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake, fake, n, nullptr) ==
        MLA_ERR_PLAN_MISMATCH);
  CHECK(mla_decode(plan, fake + 2, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake, fake, n,
                   nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_decode_stages(plan, fake, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake, fake, n,
                          nullptr, 7) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_decode(plan, fake, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake, fake, n - 256,
                   nullptr) == MLA_ERR_WORKSPACE_TOO_SMALL);
  CHECK(mla_debug_gather(plan, nullptr, (int32_t*)fake, fake, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  int32_t segs[4];
  CHECK(mla_plan_get_segments(plan, segs, 0, nullptr, 0) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_read_status(nullptr, nullptr, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  mla_plan_destroy(plan);
  mla_plan_destroy(nullptr);
  // shapes at the edges of int32 and of the supported set
  p.max_pages_per_seq = 1 << 30;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_ERR_UNSUPPORTED);
  p.max_pages_per_seq = 2;
  p.num_heads = 272;
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_ERR_UNSUPPORTED);
  p.num_heads = 16;
  lens[1] = 129;   // > max_pages_per_seq * page_size
  CHECK(mla_plan(&p, lens, &opt, &plan) == MLA_ERR_INVALID_ARGUMENT);
  lens[1] = 50;
  CHECK(mla_devplan_workspace_bytes(&p, 256) > 0 && mla_devplan_workspace_bytes(&p, -1) == 0);
  const size_t dn = mla_devplan_workspace_bytes(&p, 256);
  CHECK(mla_devplan_prepare(&p, 256, fake, dn - 1, nullptr) == MLA_ERR_WORKSPACE_TOO_SMALL);
  CHECK(mla_decode_devplan(&p, 256, fake + 8, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake, fake,
                           dn, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  // the entry point without a workspace: a schedule larger than its scratch is refused first
  CHECK(mla_decode_devplan_noalloc(&p, 1 << 20, fake, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake,
                                   (float*)fake, nullptr) == MLA_ERR_WORKSPACE_TOO_SMALL);
  CHECK(mla_decode_devplan_noalloc(&p, -1, fake, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake, (float*)fake,
                                   nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_decode_devplan_noalloc(&p, 256, nullptr, fake, (int32_t*)fake, (int32_t*)fake, 0.1f, fake,
                                   (float*)fake, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_decode_devplan_noalloc(&p, 256, fake, fake, (int32_t*)fake, (int32_t*)fake, __builtin_inff(), fake,
                                   (float*)fake, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_q_absorb(&p, nullptr, fake, fake, (int32_t*)fake, 10000.f, fake, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_kv_append(&p, fake, fake, (int32_t*)fake, (int32_t*)fake, -1.f, fake, nullptr, nullptr) ==
        MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_out_absorb(&p, fake + 8, fake, fake, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  for (int s = -1; s < 8; ++s) CHECK(mla_status_string((mla_status_t)s) != nullptr);
  CHECK(mla_stream_probe(nullptr, 1 << 20, 256, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_stream_probe(fake + 16, 1 << 30, 256, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  CHECK(mla_stream_probe(fake, 1000, 256, nullptr) == MLA_ERR_INVALID_ARGUMENT);
  return true;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 400;
  if (!validation_paths()) return 1;
  for (int i = 0; i < iters; ++i)
    if (!fuzz_one(i)) {
      std::printf("fuzz iteration %d failed\n", i);
      return 1;
    }
  std::printf("ok\n");
  return 0;
}
