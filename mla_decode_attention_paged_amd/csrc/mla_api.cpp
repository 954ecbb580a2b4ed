// C-ABI entry points: argument validation, workspace layout, launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include <unistd.h>

#include "mla.h"
#include "mla_internal.h"

struct mla_plan_s {
  mla::PlanImpl impl;
};

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status_t check_problem(const mla_problem_t* p) {
  if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
  if (p->q_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "q_len must be >= 1 (got %d)", p->q_len);
  if (p->num_heads < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_heads must be >= 1 (got %d)", p->num_heads);
  if (p->page_size < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "page_size must be >= 1 (got %d)", p->page_size);
  if (p->num_pages < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be >= 0 (got %d)", p->num_pages);
  if (p->max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq must be >= 1 (got %d)", p->max_pages_per_seq);
  if (p->out_dtype != MLA_DTYPE_BF16 && p->out_dtype != MLA_DTYPE_FP32)
    return fail(MLA_ERR_INVALID_ARGUMENT, "out_dtype must be MLA_DTYPE_BF16 or MLA_DTYPE_FP32");
  if (p->causal != 0 && p->causal != 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", p->causal);
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_dtype must be MLA_KV_BF16 or MLA_KV_FP8_E4M3");
  if (p->head_dim_qk != mla::kDqk || p->head_dim_v != mla::kDv)
    return fail(MLA_ERR_UNSUPPORTED, "head dims must be 576/512 (got %d/%d)", p->head_dim_qk, p->head_dim_v);
  if (p->page_size % mla::kBlock != 0)
    return fail(MLA_ERR_UNSUPPORTED, "page_size must be a multiple of 16 (got %d)", p->page_size);
  const int64_t R = (int64_t)p->q_len * p->num_heads;
  if (R % 16 != 0 || R > mla::kMaxRows)
    return fail(MLA_ERR_UNSUPPORTED, "q_len*num_heads must be a multiple of 16 and <= 256 (got %lld)",
                (long long)R);
  if ((int64_t)p->max_pages_per_seq * p->page_size > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "max_pages_per_seq * page_size exceeds int32");
  return MLA_OK;
}

mla_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Plan ids: unique within the process and unlikely to repeat across processes (a salt from
// the process id and the clock in the high half); never zero, so a cleared workspace
// matches no plan.
uint64_t next_plan_id() {
  static const uint64_t salt =
      ((uint64_t)getpid() << 40) ^ (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  static std::atomic<uint64_t> counter{0};
  uint64_t id = (salt << 20) ^ (counter.fetch_add(1) + 1);
  return id ? id : 1;
}

// Which plan each workspace address last received with mla_plan_upload (host side).
std::mutex g_ws_mu;
std::unordered_map<uintptr_t, uint64_t> g_ws_plan;

void register_upload(const void* ws, uint64_t id) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  g_ws_plan[(uintptr_t)ws] = id;
}

bool holds_plan(const void* ws, uint64_t id) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws_plan.find((uintptr_t)ws);
  return it != g_ws_plan.end() && it->second == id;
}

void forget_plan(uint64_t id) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto it = g_ws_plan.begin(); it != g_ws_plan.end();) {
    if (it->second == id)
      it = g_ws_plan.erase(it);
    else
      ++it;
  }
}

// Device-scheduled decode: workers per row group and the workspace layout
// [status | per-sequence cut (4 x batch + 2 int32) | partial lse (2W x R) | partial out (2W x R x 512)].
struct DevLayout {
  int32_t workers = 0, row_groups = 0;
  size_t off_info = 0, off_cnt = 0, off_lse = 0, off_o = 0, bytes = 0;
};

mla_status_t dev_layout(const mla_problem_t* p, int32_t num_workers, DevLayout& d) {
  mla_status_t s = check_problem(p);
  if (s != MLA_OK) return s;
  if (num_workers < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_workers must be >= 0");
  const int32_t R = p->q_len * p->num_heads;
  d.row_groups = R / 16;
  int32_t w = num_workers;
  if (w == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice (pass num_workers to size without a device)");
    hipDeviceProp_t pr;
    e = hipGetDeviceProperties(&pr, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    w = pr.multiProcessorCount / d.row_groups;
  }
  d.workers = w < 1 ? 1 : w;
  d.off_info = mla::kMetaOffset;
  // per (sequence, row group) piece counters of the combining launch: cleared by
  // mla_devplan_prepare, left at zero by every combining launch
  d.off_cnt = align256(d.off_info + 4 * (4 * (size_t)p->batch + 2));
  d.off_lse = align256(d.off_cnt + 4 * (size_t)p->batch * d.row_groups);
  d.off_o = align256(d.off_lse + 4 * 2 * (size_t)d.workers * R);
  d.bytes = align256(d.off_o + 4 * 2 * (size_t)d.workers * R * mla::kDv);
  return MLA_OK;
}

// Pointer and scale checks shared by the device-scheduled entry points.
mla_status_t check_devplan_args(const void* q, const void* kv_cache, const int32_t* block_table,
                                const int32_t* cache_seqlens, float softmax_scale, const void* out, const float* lse) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)q % 16 || (uintptr_t)kv_cache % 16 || (uintptr_t)out % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q, kv_cache and out must be 16-B aligned");
  if ((uintptr_t)block_table % 4 || (uintptr_t)cache_seqlens % 4 || (uintptr_t)lse % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "block_table, cache_seqlens and lse must be 4-B aligned");
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_PLAN_MISMATCH: return "plan does not match the call";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status_t mla_plan(const mla_problem_t* problem, const int32_t* cache_seqlens_host,
                      const mla_plan_options_t* options, mla_plan_t* plan_out) {
  if (!plan_out) return fail(MLA_ERR_INVALID_ARGUMENT, "plan_out is NULL");
  *plan_out = nullptr;
  mla_status_t s = check_problem(problem);
  if (s != MLA_OK) return s;
  if (!cache_seqlens_host) return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seqlens_host is NULL");
  mla_plan_options_t opt{};
  if (options) opt = *options;
  for (int i = 0; i < 5; ++i)
    if (opt.reserved[i] != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "options.reserved must be zero");
  {
    const int32_t rpg = opt.rows_per_group, R = problem->q_len * problem->num_heads;
    if (rpg != 0 && rpg != 16 && rpg != 32 && rpg != 64 && rpg != 128)
      return fail(MLA_ERR_INVALID_ARGUMENT, "options.rows_per_group must be 0, 16, 32, 64 or 128");
    if (rpg > 16 && R % rpg != 0)
      return fail(MLA_ERR_UNSUPPORTED, "rows_per_group %d needs R a multiple of it", rpg);
    if (rpg == 32 && problem->kv_dtype == MLA_KV_FP8_E4M3)
      return fail(MLA_ERR_UNSUPPORTED, "rows_per_group 32 needs a bf16 cache (fp8 rows: 16, 64 or 128)");
  }
  if (opt.num_cus < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "options.num_cus must be >= 0");
  if (opt.force_splits < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "options.force_splits must be >= 0");
  const int64_t cap = (int64_t)problem->max_pages_per_seq * problem->page_size;
  for (int b = 0; b < problem->batch; ++b) {
    int32_t L = cache_seqlens_host[b];
    if (L < 0 || L > cap)
      return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seqlens[%d] = %d outside [0, %lld]", b, L, (long long)cap);
    if (L > 0 && problem->num_pages == 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seqlens[%d] = %d but num_pages is 0", b, L);
  }
  int32_t cus = opt.num_cus;
  if (cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice (set options.num_cus to plan without a device)");
    hipDeviceProp_t pr;
    e = hipGetDeviceProperties(&pr, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    cus = pr.multiProcessorCount;
  }
  mla_plan_s* pl = new (std::nothrow) mla_plan_s();
  if (!pl) return fail(MLA_ERR_INVALID_ARGUMENT, "out of host memory");
  std::string err;
  s = mla::build_plan(*problem, cache_seqlens_host, cus, opt.force_splits, opt.rows_per_group, next_plan_id(),
                      pl->impl, err);
  if (s != MLA_OK) {
    delete pl;
    return fail(s, "%s", err.c_str());
  }
  *plan_out = pl;
  return MLA_OK;
}

mla_status_t mla_plan_get_info(mla_plan_t plan, mla_plan_info_t* info) {
  if (!plan || !info) return fail(MLA_ERR_INVALID_ARGUMENT, "plan or info is NULL");
  const mla::PlanImpl& p = plan->impl;
  mla_plan_info_t r{};
  r.num_workers = p.num_workers;
  r.grid_size = p.grid;
  r.num_segments = (int32_t)p.pieces.size();
  r.num_partials = p.num_partials;
  r.num_combine = (int32_t)p.merges.size();
  r.rows_per_group = p.rows_per_group;
  r.row_groups = p.row_groups;
  r.granule = p.granule;
  int64_t mx = 0, mn = INT64_MAX;
  for (int64_t c : p.worker_cost) {
    mx = c > mx ? c : mx;
    mn = c < mn ? c : mn;
  }
  r.max_worker_cost = mx;
  r.min_worker_cost = p.worker_cost.empty() ? 0 : mn;
  r.metadata_bytes = (int64_t)p.meta_end;
  r.workspace_bytes = (int64_t)p.ws_bytes;
  *info = r;
  return MLA_OK;
}

mla_status_t mla_plan_get_segments(mla_plan_t plan, int32_t* segments, int64_t segments_capacity,
                                   int32_t* worker_offsets, int64_t offsets_capacity) {
  if (!plan || !segments) return fail(MLA_ERR_INVALID_ARGUMENT, "plan or segments is NULL");
  const mla::PlanImpl& p = plan->impl;
  if (segments_capacity < 4 * (int64_t)p.pieces.size())
    return fail(MLA_ERR_INVALID_ARGUMENT, "segments capacity %lld < %lld", (long long)segments_capacity,
                (long long)(4 * p.pieces.size()));
  if (worker_offsets && offsets_capacity < (int64_t)p.worker_off.size())
    return fail(MLA_ERR_INVALID_ARGUMENT, "worker_offsets capacity too small");
  for (size_t i = 0; i < p.pieces.size(); ++i) {
    segments[4 * i + 0] = p.pieces[i].seq;
    segments[4 * i + 1] = p.pieces[i].tok_begin;
    segments[4 * i + 2] = p.pieces[i].tok_end;
    segments[4 * i + 3] = p.pieces[i].slot;
  }
  if (worker_offsets)
    for (size_t i = 0; i < p.worker_off.size(); ++i) worker_offsets[i] = p.worker_off[i];
  return MLA_OK;
}

size_t mla_plan_workspace_bytes(mla_plan_t plan) { return plan ? plan->impl.ws_bytes : 0; }

mla_status_t mla_plan_upload(mla_plan_t plan, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-B aligned");
  if (workspace_bytes < plan->impl.ws_bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < required %zu B", workspace_bytes,
                plan->impl.ws_bytes);
  hipError_t e = hipMemcpyAsync(workspace, plan->impl.meta_host.data(), plan->impl.meta_end,
                                hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan upload)");
  register_upload(workspace, plan->impl.plan_id);
  return MLA_OK;
}

mla_status_t mla_decode(mla_plan_t plan, const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_stages(plan, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse, workspace,
                           workspace_bytes, stream, MLA_STAGE_ALL);
}

mla_status_t mla_decode_stages(mla_plan_t plan, const void* q, const void* kv_cache, const int32_t* block_table,
                               const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream, uint32_t stages) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (stages != MLA_STAGE_COMBINED && (stages == 0 || (stages & ~MLA_STAGE_ALL) != 0))
    return fail(MLA_ERR_INVALID_ARGUMENT, "stages must be a non-empty subset of MLA_STAGE_ALL, or MLA_STAGE_COMBINED");
  const mla::PlanImpl& p = plan->impl;
  if (stages == MLA_STAGE_COMBINED && p.rows_per_group != 16)
    return fail(MLA_ERR_UNSUPPORTED, "MLA_STAGE_COMBINED runs the 16-row kernel (this plan has %d rows per group)",
                p.rows_per_group);
  if (!q || !kv_cache || !block_table || !cache_seqlens || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)q % 16 || (uintptr_t)kv_cache % 16 || (uintptr_t)out % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q, kv_cache and out must be 16-B aligned");
  if ((uintptr_t)block_table % 4 || (uintptr_t)cache_seqlens % 4 || (uintptr_t)lse % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "block_table, cache_seqlens and lse must be 4-B aligned");
  if ((uintptr_t)workspace % 256 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-B aligned");
  if (workspace_bytes < p.ws_bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < required %zu B", workspace_bytes, p.ws_bytes);
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if (!holds_plan(workspace, p.plan_id))
    return fail(MLA_ERR_PLAN_MISMATCH, "workspace %p last received another plan's schedule, or none "
                "(mla_plan_upload this plan into it first)", workspace);

  char* ws = (char*)workspace;
  mla::DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kv = (const uint16_t*)kv_cache;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.worker_off = (const int32_t*)(ws + p.off_worker);
  a.pieces = (const int32_t*)(ws + p.off_pieces);
  a.out = out;
  a.lse = lse;
  a.part_lse = (float*)(ws + p.off_lse);
  a.part_o = (float*)(ws + p.off_o);
  a.status = (int32_t*)ws;
  a.ws_plan_id = (const uint64_t*)(ws + mla::kPlanIdOffset);
  a.plan_id = p.plan_id;
  a.plan_len = (const int32_t*)(ws + p.off_lens);
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  a.rows = p.rows;
  a.page_size = p.prob.page_size;
  a.page_shift = mla::page_shift_of(p.prob.page_size);
  a.num_pages = p.prob.num_pages;
  a.bt_stride = p.prob.max_pages_per_seq;
  a.num_workers = p.num_workers;
  a.row_groups = p.row_groups;
  a.q_len = p.prob.q_len;
  a.num_heads = p.prob.num_heads;
  a.causal = p.prob.causal;
  a.kv_fp8 = p.prob.kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0;
  const bool f32 = p.prob.out_dtype == MLA_DTYPE_FP32;
  if (stages == MLA_STAGE_COMBINED) {
    if (p.grid == 0) return MLA_OK;
    a.merge_cnt = (int32_t*)(ws + p.off_cnt);
    a.seq_merge = (const int32_t*)(ws + p.off_seqm);
    int e = mla::launch_decode(a, p.rows_per_group, f32, p.grid, stream);
    if (e) return fail(MLA_ERR_HIP, "combining split-decode launch: %s", mla::hip_error_string(e));
    return MLA_OK;
  }
  if ((stages & MLA_STAGE_SPLIT) && p.grid > 0) {
    int e = mla::launch_decode(a, p.rows_per_group, f32, p.grid, stream);
    if (e) return fail(MLA_ERR_HIP, "split-decode launch: %s", mla::hip_error_string(e));
  }
  if ((stages & MLA_STAGE_MERGE) && !p.merges.empty()) {
    mla::MergeArgs m{};
    m.merges = (const int32_t*)(ws + p.off_merges);
    m.ws_plan_id = a.ws_plan_id;
    m.plan_id = p.plan_id;
    m.part_lse = a.part_lse;
    m.part_o = a.part_o;
    m.out = out;
    m.lse = lse;
    m.rows = p.rows;
    m.num_merges = (int32_t)p.merges.size();
    m.uniform_ns = p.merge_uniform;
    m.max_ns = p.merge_max_ns;
    int e = mla::launch_merge(m, f32, stream);
    if (e) return fail(MLA_ERR_HIP, "merge launch: %s", mla::hip_error_string(e));
  }
  return MLA_OK;
}

mla_status_t mla_debug_gather(mla_plan_t plan, const void* kv_cache, const int32_t* block_table, void* rows_out,
                              void* stream) {
  if (!plan || !kv_cache || !block_table || !rows_out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)kv_cache % 16 || (uintptr_t)rows_out % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_cache and rows_out must be 16-B aligned");
  const mla::PlanImpl& p = plan->impl;
  for (int b = 0; b < p.prob.batch; ++b) {
    if (p.seqlens[b] == 0) continue;
    const int32_t row_bytes = p.prob.kv_dtype == MLA_KV_FP8_E4M3 ? mla::kRowBytesFp8 : mla::kRowBytesBf16;
    int e = mla::launch_gather(kv_cache, block_table, rows_out, b, p.seqlens[b], p.row_offsets[b],
                               p.prob.page_size, p.prob.max_pages_per_seq, p.prob.num_pages, row_bytes, stream);
    if (e) return fail(MLA_ERR_HIP, "gather launch: %s", mla::hip_error_string(e));
  }
  return MLA_OK;
}

size_t mla_devplan_workspace_bytes(const mla_problem_t* problem, int32_t num_workers) {
  DevLayout d;
  return dev_layout(problem, num_workers, d) == MLA_OK ? d.bytes : 0;
}

mla_status_t mla_devplan_prepare(const mla_problem_t* problem, int32_t num_workers, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  DevLayout d;
  mla_status_t s = dev_layout(problem, num_workers, d);
  if (s != MLA_OK) return s;
  if (!workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-B aligned");
  if (workspace_bytes < d.bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < required %zu B", workspace_bytes, d.bytes);
  int e = mla::launch_fill_zero(workspace, d.off_lse, stream);
  if (e) return fail(MLA_ERR_HIP, "workspace clear: %s", mla::hip_error_string(e));
  return MLA_OK;
}

namespace {
mla_status_t devplan_decode(const mla_problem_t* problem, int32_t num_workers, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                            bool combined) {
  DevLayout d;
  mla_status_t s = dev_layout(problem, num_workers, d);
  if (s != MLA_OK) return s;
  s = check_devplan_args(q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse);
  if (s != MLA_OK) return s;
  if (!workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-B aligned");
  if (workspace_bytes < d.bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < required %zu B", workspace_bytes, d.bytes);
  const mla_problem_t& p = *problem;
  char* ws = (char*)workspace;
  mla::DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kv = (const uint16_t*)kv_cache;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.out = out;
  a.lse = lse;
  a.part_lse = (float*)(ws + d.off_lse);
  a.part_o = (float*)(ws + d.off_o);
  a.status = (int32_t*)ws;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  a.rows = p.q_len * p.num_heads;
  a.page_size = p.page_size;
  a.page_shift = mla::page_shift_of(p.page_size);
  a.num_pages = p.num_pages;
  a.bt_stride = p.max_pages_per_seq;
  a.num_workers = d.workers;
  a.row_groups = d.row_groups;
  a.q_len = p.q_len;
  a.num_heads = p.num_heads;
  a.causal = p.causal;
  a.kv_fp8 = p.kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0;
  a.batch = p.batch;
  a.seq_info = (int32_t*)(ws + d.off_info);
  const int32_t grid = d.row_groups > 1 ? (d.workers + 7) / 8 * 8 * d.row_groups : d.workers;
  const bool f32 = p.out_dtype == MLA_DTYPE_FP32;
  if (combined) a.merge_cnt = (int32_t*)(ws + d.off_cnt);
  int e = mla::launch_decode(a, 16, f32, grid, stream, true);
  if (e) return fail(MLA_ERR_HIP, "device-scheduled decode launch: %s", mla::hip_error_string(e));
  if (combined) return MLA_OK;
  mla::MergeArgs m{};
  m.part_lse = a.part_lse;
  m.part_o = a.part_o;
  m.out = out;
  m.lse = lse;
  m.rows = a.rows;
  m.seq_info = a.seq_info;
  m.batch = p.batch;
  e = mla::launch_merge_dev(m, f32, stream);
  if (e) return fail(MLA_ERR_HIP, "device-scheduled merge launch: %s", mla::hip_error_string(e));
  return MLA_OK;
}
}  // namespace

mla_status_t mla_decode_devplan(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                                float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return devplan_decode(problem, num_workers, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse,
                        workspace, workspace_bytes, stream, false);
}

mla_status_t mla_decode_devplan_combined(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                         const void* kv_cache, const int32_t* block_table,
                                         const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return devplan_decode(problem, num_workers, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse,
                        workspace, workspace_bytes, stream, true);
}

mla_status_t mla_decode_devplan_noalloc(const mla_problem_t* problem, int32_t num_workers, const void* q,
                                        const void* kv_cache, const int32_t* block_table,
                                        const int32_t* cache_seqlens, float softmax_scale, void* out, float* lse,
                                        void* stream) {
  DevLayout d;
  mla_status_t s = dev_layout(problem, num_workers, d);
  if (s != MLA_OK) return s;
  s = check_devplan_args(q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse);
  if (s != MLA_OK) return s;
  if (d.bytes > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "the device schedule needs %zu B of scratch; the library holds %u B per GPU", d.bytes,
                (unsigned)MLA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const int e = mla::noalloc_scratch(&ws);
  if (e) return fail(MLA_ERR_HIP, "scratch address: %s", mla::hip_error_string(e));
  return mla_decode_devplan(problem, num_workers, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse,
                            ws, MLA_NOALLOC_SCRATCH_BYTES, stream);
}

mla_status_t mla_stream_probe(const void* buffer, size_t bytes, int32_t num_workgroups, void* stream) {
  if (!buffer) return fail(MLA_ERR_INVALID_ARGUMENT, "buffer is NULL");
  if ((uintptr_t)buffer % 1024) return fail(MLA_ERR_INVALID_ARGUMENT, "buffer must be 1 KiB aligned");
  if (num_workgroups < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_workgroups must be >= 1");
  const int64_t per_wg = (int64_t)(bytes / (size_t)num_workgroups) / mla::kProbeUnit * mla::kProbeUnit;
  if (per_wg == 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must cover at least %lld per work-group", (long long)mla::kProbeUnit);
  const int e = mla::launch_stream_probe(buffer, per_wg, num_workgroups, stream);
  if (e) return fail(MLA_ERR_HIP, "stream probe launch: %s", mla::hip_error_string(e));
  return MLA_OK;
}

mla_status_t mla_read_status(const void* workspace, void* stream, int32_t* status_out) {
  if (!workspace || !status_out) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace or status_out is NULL");
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, workspace, sizeof v, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (status)");
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (status)");
  *status_out = v;
  return MLA_OK;
}

mla_status_t mla_q_absorb(const mla_problem_t* problem, const void* q_nope, const void* q_pe, const void* w_uk,
                          const int32_t* positions, float rope_base, void* q_out, void* stream) {
  mla_status_t s = check_problem(problem);
  if (s != MLA_OK) return s;
  if (!q_nope || !q_pe || !w_uk || !positions || !q_out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)q_nope % 16 || (uintptr_t)w_uk % 16 || (uintptr_t)q_out % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_nope, w_uk and q_out must be 16-B aligned");
  if ((uintptr_t)q_pe % 4 || (uintptr_t)positions % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_pe and positions must be 4-B aligned");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope_base must be a finite positive number");
  mla::LayerArgs a{};
  a.batch = problem->batch;
  a.q_len = problem->q_len;
  a.num_heads = problem->num_heads;
  a.rope_base = rope_base;
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.w_uk = w_uk;
  a.positions = positions;
  a.q_out = q_out;
  int e = mla::launch_q_absorb(a, stream);
  if (e) return fail(MLA_ERR_HIP, "query absorption launch: %s", mla::hip_error_string(e));
  return MLA_OK;
}

mla_status_t mla_kv_append(const mla_problem_t* problem, const void* c_kv, const void* k_pe,
                           const int32_t* positions, const int32_t* block_table, float rope_base, void* kv_cache,
                           int32_t* status, void* stream) {
  mla_status_t s = check_problem(problem);
  if (s != MLA_OK) return s;
  if (!c_kv || !k_pe || !positions || !block_table || !kv_cache)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)c_kv % 16 || (uintptr_t)kv_cache % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "c_kv and kv_cache must be 16-B aligned");
  if ((uintptr_t)k_pe % 4 || (uintptr_t)positions % 4 || (uintptr_t)block_table % 4 || (uintptr_t)status % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "k_pe, positions, block_table and status must be 4-B aligned");
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope_base must be a finite positive number");
  mla::LayerArgs a{};
  a.batch = problem->batch;
  a.q_len = problem->q_len;
  a.num_heads = problem->num_heads;
  a.page_size = problem->page_size;
  a.num_pages = problem->num_pages;
  a.max_pages_per_seq = problem->max_pages_per_seq;
  a.kv_fp8 = problem->kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 0;
  a.rope_base = rope_base;
  a.c_kv = c_kv;
  a.k_pe = k_pe;
  a.positions = positions;
  a.block_table = block_table;
  a.kv_cache = kv_cache;
  a.status = status;
  int e = mla::launch_kv_append(a, stream);
  if (e) return fail(MLA_ERR_HIP, "cache append launch: %s", mla::hip_error_string(e));
  return MLA_OK;
}

mla_status_t mla_out_absorb(const mla_problem_t* problem, const void* out_latent, const void* w_uv, void* o,
                            void* stream) {
  mla_status_t s = check_problem(problem);
  if (s != MLA_OK) return s;
  if (!out_latent || !w_uv || !o) return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((uintptr_t)out_latent % 16 || (uintptr_t)w_uv % 16 || (uintptr_t)o % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "out_latent, w_uv and o must be 16-B aligned");
  mla::LayerArgs a{};
  a.batch = problem->batch;
  a.q_len = problem->q_len;
  a.num_heads = problem->num_heads;
  a.out_latent = out_latent;
  a.w_uv = w_uv;
  a.o = o;
  const bool f32 = problem->out_dtype == MLA_DTYPE_FP32;
  int e = mla::launch_out_absorb(a, f32, f32, stream);
  if (e) return fail(MLA_ERR_HIP, "output projection launch: %s", mla::hip_error_string(e));
  return MLA_OK;
}

void mla_plan_destroy(mla_plan_t plan) {
  if (!plan) return;
  forget_plan(plan->impl.plan_id);
  delete plan;
}

}  // extern "C"
