// Internal declarations shared by the C-ABI layer, the planner and the kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "mla.h"

namespace mla {

constexpr int kDqk = 576;          // cached row width: 512 latent + 64 rope
constexpr int kDv = 512;           // latent columns, also V
constexpr int kBlock = 16;         // tokens per KV block (one MFMA M tile)
constexpr int kWaves = 4;          // waves per work-group in the split-decode kernel
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 256;   // q_len * num_heads: two query tokens over 128 heads
constexpr int kRowBytesBf16 = kDqk * 2;   // 1,152
constexpr int kRowBytesFp8 = 656;         // 512 E4M3 + 64 bf16 rope + 4 float32 scales

// Workspace layout (byte offsets from the workspace base).
//   [0, 4)                status word (int32, bits kStatus*)
//   [8, 16)               id of the plan whose schedule the workspace holds (uint64)
//   [kMetaOffset, ...)    worker offsets, pieces, merge items, the plan's lengths (int32)
//   [off_lse, ...)        partial lse   [num_partials][R] fp32
//   [off_o, ...)          partial out   [num_partials][R][512] fp32
constexpr size_t kPlanIdOffset = 8;
constexpr size_t kMetaOffset = 256;

// Bits of the workspace status word (mla_read_status).
constexpr int32_t kStatusBadPage = 1;        // a used block_table entry was outside [0, num_pages)
constexpr int32_t kStatusLongerThanPlan = 4; // a device cache_seqlens value exceeded the plan's
constexpr int32_t kStatusPlanMismatch = 8;   // the workspace held another plan's schedule: nothing ran

struct Piece {            // one (sequence, token range) handled by one work-group
  int32_t seq, tok_begin, tok_end, slot;   // slot -1: write out/lse directly
};

struct MergeItem {        // one split sequence for the merge kernel
  int32_t seq, slot_begin, num_slots, pad;
};

struct PlanImpl {
  mla_problem_t prob{};
  std::vector<int32_t> seqlens;
  std::vector<int64_t> row_offsets;        // prefix sums of seqlens (debug gather)
  int32_t num_cus = 0;
  int32_t rows = 0;                        // R
  int32_t rows_per_group = 16;             // 16 * NB
  int32_t row_groups = 1;
  int32_t granule = kBlock;
  int32_t num_workers = 0;                 // with work
  int32_t grid = 0;                        // launched work-groups
  std::vector<int32_t> worker_off;         // num_workers + 1
  std::vector<Piece> pieces;
  std::vector<MergeItem> merges;
  int32_t merge_uniform = 0;               // ns when item b merges slots [b*ns, (b+1)*ns) for every b
  int32_t merge_max_ns = 0;                // the largest number of pieces of a merged sequence
  std::vector<int64_t> worker_cost;
  int32_t num_partials = 0;
  uint64_t plan_id = 0;                    // nonzero, unique per plan in the process
  // workspace layout
  size_t off_worker = 0, off_pieces = 0, off_merges = 0, off_lens = 0, meta_end = 0;
  size_t off_seqm = 0, off_cnt = 0;        // combining in the decode launch: [B][2] slots, [B][row groups] counters
  size_t off_lse = 0, off_o = 0, ws_bytes = 0;
  std::vector<uint8_t> meta_host;          // bytes [0, meta_end) as uploaded
};

// Planner (pure host code).  Returns MLA_OK or an error with `err` filled.
mla_status_t build_plan(const mla_problem_t& p, const int32_t* seqlens, int32_t num_cus,
                        int32_t force_splits, int32_t rows_per_group, uint64_t plan_id, PlanImpl& out,
                        std::string& err);

// Parameters of the split-decode kernel.
// log2(page_size) when the page size is a power of two, else -1 (the kernels then divide)
inline int32_t page_shift_of(int32_t page_size) {
  if (page_size <= 0 || (page_size & (page_size - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) < page_size) ++s;
  return s;
}

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* worker_off;
  const int32_t* pieces;         // int32 quadruples
  void* out;
  float* lse;                    // may be null
  float* part_lse;
  float* part_o;
  int32_t* status;
  const uint64_t* ws_plan_id;    // the plan id stored in the workspace (host schedule only)
  uint64_t plan_id;              // the id of the plan this launch was made from
  const int32_t* plan_len;       // [batch] the lengths the plan was made for (host schedule only)
  float scale_log2;              // softmax_scale * log2(e)
  int32_t rows;                  // R
  int32_t page_size;
  int32_t page_shift;              // log2(page_size) for a power of two, else -1
  int32_t num_pages;
  int32_t bt_stride;
  int32_t num_workers;
  int32_t row_groups;
  int32_t q_len;
  int32_t num_heads;
  int32_t causal;                // row r = i * num_heads + h sees t < L - (q_len - 1 - i)
  int32_t kv_fp8;                // cache rows are 656-byte fp8 rows
  int32_t batch;
  int32_t* seq_info;             // device schedule: per-sequence cut [batch][4] + {T, W}
  // Combining in the decode launch (16-row kernel): null = a merge launch follows.
  int32_t* merge_cnt;            // [batch][row_groups] pieces done, zero between calls
  const int32_t* seq_merge;      // host schedule: [batch][2] first slot and number of pieces
};

struct MergeArgs {
  const int32_t* merges;         // int32 quadruples
  const uint64_t* ws_plan_id;    // host schedule: the plan id stored in the workspace (null: no check)
  uint64_t plan_id;
  const float* part_lse;
  const float* part_o;
  void* out;
  float* lse;
  int32_t rows;
  int32_t num_merges;
  int32_t uniform_ns;            // > 0: item i is sequence i with slots [i*ns, (i+1)*ns)
  int32_t max_ns;                // the largest piece count of a merged sequence (batch size)
  const int32_t* seq_info;       // device schedule (merge_dev_kernel)
  int32_t batch;
};

// Parameters of the steps around the decode (mla_layer_kernels.hip).
struct LayerArgs {
  int32_t batch, q_len, num_heads;
  int32_t page_size, num_pages, max_pages_per_seq;   // kv append
  int32_t kv_fp8;
  float rope_base;
  const void* q_nope;            // [B, q_len, H, 128] bf16
  const void* q_pe;              // [B, q_len, H, 64] bf16
  const void* w_uk;              // [H, 512, 128] bf16
  const int32_t* positions;      // [B, q_len]
  void* q_out;                   // [B, q_len, H, 576] bf16
  const void* c_kv;              // [B, q_len, 512] bf16
  const void* k_pe;              // [B, q_len, 64] bf16
  const int32_t* block_table;
  void* kv_cache;
  int32_t* status;               // may be null
  const void* out_latent;        // [B, q_len, H, 512] bf16 or fp32
  const void* w_uv;              // [H, 128, 512] bf16
  void* o;                       // [B, q_len, H, 128] bf16 or fp32
};

int launch_q_absorb(const LayerArgs& a, void* stream);
int launch_kv_append(const LayerArgs& a, void* stream);
int launch_out_absorb(const LayerArgs& a, bool in_f32, bool out_f32, void* stream);

// Kernel launchers (mla_kernels.hip).  Return a HIP error code (0 = success).
int launch_decode(const DecodeArgs& a, int rows_per_group, bool out_fp32, int grid, void* stream,
                  bool device_schedule = false);
int launch_merge_dev(const MergeArgs& a, bool out_fp32, void* stream);
int launch_fill_zero(void* p, size_t bytes, void* stream);   // bytes: a multiple of 4
int launch_merge(const MergeArgs& a, bool out_fp32, void* stream);
int launch_stream_probe(const void* buf, int64_t per_wg, int grid, void* stream);
constexpr int64_t kProbeUnit = (int64_t)kWaves * kBlock * kDqk * 2;   // 73,728: one 18 KB block per wave
int launch_gather(const void* kv, const int32_t* block_table, void* rows_out, int32_t seq, int32_t length,
                  int64_t row_offset, int32_t page_size, int32_t bt_stride, int32_t num_pages, int32_t row_bytes,
                  void* stream);
const char* hip_error_string(int code);
// Device address of this GPU's scratch array (MLA_NOALLOC_SCRATCH_BYTES) for the entry point that
// allocates nothing; looked up once per device.  Returns a HIP error code (0 = success).
int noalloc_scratch(void** out);

}  // namespace mla
