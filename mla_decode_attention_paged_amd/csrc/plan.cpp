// Split-KV planner: cuts each sequence's context into pieces so that every
// work-group of the split-decode launch gets about the same amount of work.
//
// Cost model (units: 16-token KV blocks, 18,432 bytes each):
//   a piece of n blocks costs n + kPieceOverhead, where the overhead stands for
//   loading the R query rows, filling the load pipeline and writing (then, for
//   a split sequence, re-reading in the merge) one R x 512 fp32 partial result.
// Sequences are walked in order and poured into work-groups of equal budget
// ceil(total / workers); a sequence that does not fit in the rest of a budget
// is cut, and each piece pays the overhead.  Pieces are cut on granule
// boundaries (16 tokens), so a piece never straddles a cache page
// (page_size is a multiple of 16).
#include <algorithm>
#include <cstring>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int64_t kPieceOverhead = 6;   // blocks
constexpr int64_t kMinPiece = kWaves;   // blocks: one per wave; no piece is cut smaller

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

mla_status_t build_plan(const mla_problem_t& p, const int32_t* seqlens, int32_t num_cus,
                        int32_t force_splits, int32_t rows_per_group, uint64_t plan_id, PlanImpl& pl,
                        std::string& err) {
  pl = PlanImpl{};
  pl.prob = p;
  pl.plan_id = plan_id;
  pl.num_cus = num_cus;
  const int32_t B = p.batch;
  const int64_t R = (int64_t)p.q_len * p.num_heads;
  pl.rows = (int32_t)R;
  // Query rows per work-group: 16 (the 16-row kernel, one wave per 16-token block, in R/16
  // row groups whose work-groups share a token range on one XCD), 32 (the 32-row kernel: each
  // wave takes its own 16-token blocks for all 32 rows; bf16 rows), 64 or 128 (the wide kernel:
  // four waves share each 32-token block in LDS, 32 rows per wave on 32x32x16 MFMA tiles; with
  // 64 rows two waves share each set of 32 rows and split its output columns).  When not asked
  // for: 128 if R is a multiple of 128, else 64 if R is a multiple of 64, else (bf16 rows) 32 if
  // R is a multiple of 32, else 16.  Measured on MI355X at R = 128 (ragged workload): about
  // 700-730 us with 128 rows, 1,380 us with 16; at R = 64 (batch 32 x 16K tokens) 134 us with
  // 64 rows against 168 us for a four-wave kernel with 16 rows per wave (FP8 rows: 136 us
  // against 168 us with 16 rows); at R = 32 (two-token workload, split launch) 105 us with 32
  // rows against 119 us with 16 (FP8 rows: 94 us with 16 rows against 127 us for the wide
  // kernel with four waves per 32 rows).  Larger R comes in as more row groups over the same
  // token ranges.
  const bool bf16 = p.kv_dtype != MLA_KV_FP8_E4M3;
  if (rows_per_group != 0)
    pl.rows_per_group = rows_per_group;
  else
    pl.rows_per_group = R % 128 == 0 ? 128 : R % 64 == 0 ? 64 : (R % 32 == 0 && bf16) ? 32 : 16;
  pl.row_groups = (int32_t)(R / pl.rows_per_group);
  pl.granule = kBlock;

  pl.seqlens.assign(seqlens, seqlens + B);
  pl.row_offsets.resize(B + 1);
  pl.row_offsets[0] = 0;
  for (int b = 0; b < B; ++b) pl.row_offsets[b + 1] = pl.row_offsets[b] + seqlens[b];

  std::vector<int64_t> nblk(B);
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    nblk[b] = (seqlens[b] + kBlock - 1) / kBlock;
    total += nblk[b] + kPieceOverhead;
  }

  // pieces grouped by worker
  std::vector<std::vector<Piece>> per_worker;
  std::vector<int64_t> cost;
  auto add_piece = [&](int w, int32_t b, int64_t blk0, int64_t blk1) {
    if ((int)per_worker.size() <= w) {
      per_worker.resize(w + 1);
      cost.resize(w + 1, 0);
    }
    Piece pc;
    pc.seq = b;
    pc.tok_begin = (int32_t)(blk0 * kBlock);
    pc.tok_end = (int32_t)std::min<int64_t>(seqlens[b], blk1 * kBlock);
    pc.slot = -1;
    per_worker[w].push_back(pc);
    cost[w] += (blk1 - blk0) + kPieceOverhead;
  };

  if (force_splits > 0) {
    int w = 0;
    for (int b = 0; b < B; ++b) {
      int64_t n = nblk[b];
      int64_t k = std::max<int64_t>(1, std::min<int64_t>(force_splits, n));
      for (int64_t i = 0; i < k; ++i) {
        int64_t a = n * i / k, e = n * (i + 1) / k;
        add_piece(w++, b, a, e);
      }
    }
  } else {
    int64_t workers = num_cus;
    if (pl.row_groups > 1) workers = std::max<int64_t>(1, num_cus / pl.row_groups);
    workers = std::max<int64_t>(1, workers);
    // Greedy pour with a given per-work-group budget; returns the number of
    // work-groups it needs (cutting a sequence adds one more overhead, so the
    // smallest budget that fits is found by bisection below).
    auto pour = [&](int64_t budget, bool emit) -> int64_t {
      int64_t w = 0, left = budget;
      bool fresh = true;
      for (int b = 0; b < B; ++b) {
        int64_t pos = 0, n = nblk[b];
        if (n == 0) {                                   // empty context: one empty piece
          if (emit) add_piece((int)std::min<int64_t>(w, workers - 1), b, 0, 0);
          left -= kPieceOverhead;
          fresh = false;
          if (left <= 0) { ++w; left = budget; fresh = true; }
          continue;
        }
        while (pos < n) {
          int64_t room = left - kPieceOverhead;
          if (room < kMinPiece && !fresh) { ++w; left = budget; fresh = true; continue; }
          int64_t take = std::min<int64_t>(n - pos, std::max<int64_t>(room, 1));
          if (emit && w >= workers - 1) take = n - pos;   // the last work-group takes any rest
          if (n - pos - take > 0 && n - pos - take < kMinPiece) take = n - pos;   // no slivers
          if (emit) add_piece((int)std::min<int64_t>(w, workers - 1), b, pos, pos + take);
          pos += take;
          left -= take + kPieceOverhead;
          fresh = false;
          if (left <= 0) { ++w; left = budget; fresh = true; }
        }
      }
      return fresh ? w : w + 1;
    };
    int64_t lo = std::max<int64_t>(kMinPiece + kPieceOverhead, (total + workers - 1) / workers);
    int64_t hi = std::max<int64_t>(lo, total);
    while (lo < hi) {
      int64_t mid = lo + (hi - lo) / 2;
      if (pour(mid, false) <= workers) hi = mid; else lo = mid + 1;
    }
    pour(lo, true);
  }

  // flatten, assign partial slots
  pl.num_workers = (int32_t)per_worker.size();
  std::vector<int32_t> splits(B, 0);
  for (auto& v : per_worker)
    for (auto& pc : v) splits[pc.seq]++;
  std::vector<int32_t> first_slot(B, -1);
  int32_t slots = 0;
  for (int b = 0; b < B; ++b) {
    if (splits[b] > 1) {
      first_slot[b] = slots;
      MergeItem mi{b, slots, splits[b], 0};
      pl.merges.push_back(mi);
      slots += splits[b];
      pl.merge_max_ns = std::max(pl.merge_max_ns, splits[b]);
    }
  }
  pl.num_partials = slots;
  // every sequence split into the same number of pieces: the merge kernel can derive its
  // items from the work-group index instead of reading them
  if (!pl.merges.empty() && (int64_t)pl.merges.size() == B) {
    const int32_t ns = pl.merges[0].num_slots;
    bool uniform = true;
    for (int b = 0; b < B; ++b) {
      const MergeItem& mi = pl.merges[b];
      if (mi.seq != b || mi.slot_begin != b * ns || mi.num_slots != ns) uniform = false;
    }
    pl.merge_uniform = uniform ? ns : 0;
  }
  std::vector<int32_t> next_slot = first_slot;
  pl.worker_off.push_back(0);
  for (auto& v : per_worker) {
    for (auto pc : v) {
      if (splits[pc.seq] > 1) pc.slot = next_slot[pc.seq]++;
      pl.pieces.push_back(pc);
    }
    pl.worker_off.push_back((int32_t)pl.pieces.size());
  }
  // pieces of one sequence are visited in token order, so slots follow token order
  pl.worker_cost = cost;

  if (pl.row_groups > 1) {
    int32_t padded = (pl.num_workers + 7) / 8 * 8;
    pl.grid = padded * pl.row_groups;
  } else {
    pl.grid = pl.num_workers;
  }

  // workspace layout
  pl.off_worker = kMetaOffset;
  pl.off_pieces = align_up(pl.off_worker + 4 * pl.worker_off.size(), 16);
  pl.off_merges = align_up(pl.off_pieces + sizeof(Piece) * pl.pieces.size(), 16);
  pl.off_lens = align_up(pl.off_merges + sizeof(MergeItem) * pl.merges.size(), 16);
  // combining in the decode launch: each sequence's first slot and number of pieces (0 when it
  // is not split), and one counter per (sequence, row group), uploaded as zeros; the kernel
  // leaves every counter at zero when its launch ends
  pl.off_seqm = align_up(pl.off_lens + 4 * (size_t)B, 16);
  pl.off_cnt = align_up(pl.off_seqm + 8 * (size_t)B, 16);
  pl.meta_end = align_up(pl.off_cnt + 4 * (size_t)B * pl.row_groups, 256);
  pl.off_lse = pl.meta_end;
  pl.off_o = align_up(pl.off_lse + 4 * (size_t)pl.num_partials * R, 256);
  pl.ws_bytes = align_up(pl.off_o + 4 * (size_t)pl.num_partials * R * kDv, 256);

  // bytes [0, meta_end) as uploaded: a cleared status word, the plan id, the schedule
  pl.meta_host.assign(pl.meta_end, 0);
  std::memcpy(pl.meta_host.data() + kPlanIdOffset, &pl.plan_id, sizeof pl.plan_id);
  std::memcpy(pl.meta_host.data() + pl.off_lens, seqlens, 4 * (size_t)B);
  std::memcpy(pl.meta_host.data() + pl.off_worker, pl.worker_off.data(), 4 * pl.worker_off.size());
  if (!pl.pieces.empty())
    std::memcpy(pl.meta_host.data() + pl.off_pieces, pl.pieces.data(), sizeof(Piece) * pl.pieces.size());
  if (!pl.merges.empty())
    std::memcpy(pl.meta_host.data() + pl.off_merges, pl.merges.data(), sizeof(MergeItem) * pl.merges.size());
  {
    std::vector<int32_t> seqm(2 * (size_t)B, 0);
    for (const MergeItem& mi : pl.merges) {
      seqm[2 * (size_t)mi.seq] = mi.slot_begin;
      seqm[2 * (size_t)mi.seq + 1] = mi.num_slots;
    }
    std::memcpy(pl.meta_host.data() + pl.off_seqm, seqm.data(), 8 * (size_t)B);
  }
  (void)err;
  return MLA_OK;
}

}  // namespace mla
