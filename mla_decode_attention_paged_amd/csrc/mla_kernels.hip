// gfx950 kernels for paged MLA decode: split decode (three kernels by query rows per
// work-group: split_decode_kernel for 16, split32_decode_kernel for 32, wide_decode_kernel for
// 64 and 128), merge of split results (merge_kernel, or inside split_decode_kernel when one
// launch is asked for), a read-only stream probe, and a debug gather that shares the decode
// kernel's page walk.
//
// Split-decode kernel, one work-group (4 waves) per piece list from the planner.
// Each wave streams its own 16-token KV blocks (blocks w, w+4, w+8, ... of a
// piece) through a private two-stage LDS ring filled by 16-byte
// global->LDS DMA loads (each instruction moves 128 contiguous bytes of 8 cache
// rows), and keeps its own online-softmax state.  A block's K and V^T operands
// are read out of LDS first, so its stage is refilled while the block is still
// being computed.  Per block it
// evaluates the transposed flow of the FlashMLA-ETAP summary ("Core
// mechanism"): S^T = K Q^T on bf16 MFMA with the 16 tokens on the M side and
// the query rows on N, then P^T = exp2(S^T - m), then O^T += V^T P^T, again
// with the latent dimension on M.  K and V are the same LDS bytes (V = the
// first 512 columns), read as MFMA A operands: K directly with 16-byte LDS
// reads, V^T with the gfx950 LDS transpose read.  At the end of a piece the
// four waves' states are merged in LDS and the result is written either to
// `out`/`lse` or, for a sequence split over several work-groups, to an fp32
// partial slot that the merge kernel reduces by the log-sum-exp rule.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
#define CST_AS __attribute__((address_space(4)))   // read-only during a launch: scalar loads

template <class T>
__device__ __forceinline__ const CST_AS T* as_const(const T* p) {
  return (const CST_AS T*)p;
}

constexpr int kKSteps = kDqk / 32;                 // 18 MFMA k-steps over the 576 columns
constexpr int kVBlocks = kDv / 16;                 // 32 output column blocks
constexpr int kBlockBytes = kBlock * kDqk * 2;     // 18,432 bytes per 16-token block
constexpr int kStages = 2;
constexpr int kSmemBytes = kWaves * kStages * kBlockBytes;   // 147,456
// FP8 cache rows: 512 E4M3 latent bytes, 64 bf16 rope values, 4 float32 group scales
constexpr int kF8Row = 656;
constexpr int kF8Units = kBlock * kF8Row / 16;                 // 656 16-B units per block
constexpr int kF8Stage = kBlock * kF8Row;                      // 10,496 bytes
constexpr int kF8Loads = (kF8Units + 63) / 64;                 // 11 DMA instructions per block
constexpr int kF8Stages = 3;                                   // fp8 stages per wave
constexpr int kF8WaveBytes = kF8Stages * kF8Stage;             // 31,488
constexpr int kSmemFp8 = kWaves * kF8WaveBytes;               // 125,952
constexpr int kLoadsPerBlock = kBlockBytes / (64 * 16);      // 18 DMA loads per wave per block
// Cache policy of the KV-cache DMA loads (the NT template argument of the dma_* helpers).
// With one row group every KV row is read by one work-group only, and the loads carry the
// non-temporal bit (`nt`): on MI355X a global->LDS stream with `nt` runs at ~6.9 TB/s
// against ~6.1 TB/s without it (read-only stream of 1.2 GB, 256 work-groups).  With several
// row groups the work-groups of one token range re-read it through their XCD's L2, and
// default-policy loads keep it there.
constexpr float kRescaleSlack = 8.0f;              // lazy rescale threshold (log2 units)
constexpr int kMinBlocks = kWaves;                 // device schedule: fewest blocks per work-group
constexpr int kMergeBatch = 16;                    // partial results read at a time when merging
constexpr float kNegBig = -1.0e30f;                // running-max start value (finite)
constexpr int kMergeStride = kDv + 4;              // floats per row in the merge buffer
// the four waves' states when a piece ends: o [4][16][kMergeStride] plus m and l [4][16]
constexpr int kMergeBytes = kWaves * 16 * (kMergeStride + 2) * 4;   // 132,608
constexpr int kSplitSmemBf16 = kSmemBytes > kMergeBytes ? kSmemBytes : kMergeBytes;
constexpr int kSplitSmemFp8 = kSmemFp8 > kMergeBytes ? kSmemFp8 : kMergeBytes;

// Physical row of logical token t of sequence b (the page walk).  Returns -1
// when the block-table entry is outside [0, num_pages).  page_shift = log2(page_size)
// when the page size is a power of two (shift and mask), else -1 (a division).
template <class TablePtr>
__device__ __forceinline__ int64_t kv_row_of(TablePtr block_table, int bt_stride, int page_size, int page_shift,
                                             int num_pages, int b, int t) {
  int pi, r;
  if (page_shift >= 0) {
    pi = t >> page_shift;
    r = t & (page_size - 1);
  } else {
    pi = t / page_size;
    r = t - pi * page_size;
  }
  const int page = block_table[(int64_t)b * bt_stride + pi];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + r;
}

// Host schedule: the workspace must hold the schedule of the plan the launch was made from
// (its id is written by the upload).  Otherwise nothing but the worker's piece range (two words
// inside the workspace, read alongside the id) is read from it: the status word gets
// kStatusPlanMismatch and every work-group returns.
__device__ __forceinline__ bool schedule_matches(const DecodeArgs& a) {
  if (*as_const(a.ws_plan_id) == a.plan_id) return true;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_or(a.status, kStatusPlanMismatch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Host schedule: the piece that ends sequence b in the plan (tok_end = the planned length)
// flags a device length beyond it (those tokens are not attended).
__device__ __forceinline__ void check_planned_length(const DecodeArgs& a, int b, int te_in, int L) {
  if (te_in == as_const(a.plan_len)[b] && L > te_in && threadIdx.x == 0)
    __hip_atomic_fetch_or(a.status, kStatusLongerThanPlan, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_max_over_groups(float x) {
  // lanes l, l^16, l^32, l^48 hold the same query row
  int xi = __float_as_int(x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  x = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  xi = __float_as_int(x);
  r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
  int xi = __float_as_int(x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  x = __int_as_float(r[0]) + __int_as_float(r[1]);
  xi = __float_as_int(x);
  r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Two fp32 -> packed bf16 (a in the low half), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Softmax weights as bf16 hi + lo (hi = bf16(p), lo = bf16(p - hi), ~16 mantissa bits):
// {hi(p0, p1), hi(p2, p3), lo(p0, p1), lo(p2, p3)}.
__device__ __forceinline__ u32x4_t split_hi_lo(float p0, float p1, float p2, float p3) {
  const uint32_t h01 = bf16x2_rne(p0, p1), h23 = bf16x2_rne(p2, p3);
  const uint32_t l01 = bf16x2_rne(p0 - __uint_as_float(h01 << 16), p1 - __uint_as_float(h01 & 0xFFFF0000u));
  const uint32_t l23 = bf16x2_rne(p2 - __uint_as_float(h23 << 16), p3 - __uint_as_float(h23 & 0xFFFF0000u));
  return u32x4_t{h01, h23, l01, l23};
}


// Row-major block layout of the split kernel (16-B units): chunk c of token t sits at
// 128 * (c / 8) + 8 * t + ((c % 8) ^ row_swz(t)).  One DMA instruction fills 8 tokens x
// 8 chunks (128 contiguous bytes of each row); the xor spreads the K reads (16 tokens x
// one chunk) and the V^T transpose reads over all LDS banks.
__device__ __forceinline__ int row_swz(int t) { return ((t & 2) << 1) | ((t & 4) >> 1); }

// LDS reads the compiler schedules and counts itself (lgkmcnt), so that reads of a block
// overlap the MFMAs of the same block.  Its stages are filled by dma_f8_block (asm): the
// compiler does not see those LDS writes, so it adds no wait for them before a read; the
// loop waits for them with an explicit s_waitcnt vmcnt.
__device__ __forceinline__ u32x2_t lds_ld64(LDS_AS const uint8_t* p) { return *(LDS_AS const u32x2_t*)p; }
__device__ __forceinline__ u32x4_t lds_ld128(LDS_AS const uint8_t* p) { return *(LDS_AS const u32x4_t*)p; }
// gfx950 LDS transpose read of 8-bit elements (see the FP8 operand layout in the kernel)
__device__ __forceinline__ u32x2_t lds_tr8(LDS_AS const uint8_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)p));
}

// One FP8 block (16 rows of 656 B, contiguous) into an LDS stage: 16 B per lane, lane l
// moving bytes 16l + 1024j for j < 10 and lanes l < 16 also 16l + 10240.  The instruction
// offset applies to the global and the LDS address alike; it stays below 4096, so the
// 1024-B steps go from three bases 4096 B apart.  The LDS base is taken from M0, which is
// saved and restored around the loads.  The block opens with s_waitcnt lgkmcnt(0): every
// LDS read issued before it (the stage's previous block) has completed before the stage is
// overwritten.
template <bool NT>
__device__ __forceinline__ void dma_f8_block(const uint8_t* row0, uint32_t voff, uint32_t lds, bool tail_lane) {
  const uint8_t* b1 = row0 + 4096;
  const uint8_t* b2 = row0 + 8192;
  uint32_t sv;
#define MLA_F8_DMA(NTS)                                                                          \
  asm volatile(                                                                                  \
      "s_waitcnt lgkmcnt(0)\n\ts_mov_b32 %0, m0\n\t"                                             \
      "s_mov_b32 m0, %2\n\ts_nop 0\n\t"                                                          \
      "global_load_lds_dwordx4 %1, %5" NTS "\n\t"                                                \
      "global_load_lds_dwordx4 %1, %5 offset:1024" NTS "\n\t"                                    \
      "global_load_lds_dwordx4 %1, %5 offset:2048" NTS "\n\t"                                    \
      "global_load_lds_dwordx4 %1, %5 offset:3072" NTS "\n\t"                                    \
      "s_mov_b32 m0, %3\n\ts_nop 0\n\t"                                                          \
      "global_load_lds_dwordx4 %1, %6" NTS "\n\t"                                                \
      "global_load_lds_dwordx4 %1, %6 offset:1024" NTS "\n\t"                                    \
      "global_load_lds_dwordx4 %1, %6 offset:2048" NTS "\n\t"                                    \
      "global_load_lds_dwordx4 %1, %6 offset:3072" NTS "\n\t"                                    \
      "s_mov_b32 m0, %4\n\ts_nop 0\n\t"                                                          \
      "global_load_lds_dwordx4 %1, %7" NTS "\n\t"                                                \
      "global_load_lds_dwordx4 %1, %7 offset:1024" NTS "\n\t"                                    \
      "s_mov_b32 m0, %0"                                                                         \
      : "=&s"(sv)                                                                                \
      : "v"(voff), "s"(lds), "s"(lds + 4096), "s"(lds + 8192), "s"(row0), "s"(b1), "s"(b2)      \
      : "memory")
#define MLA_F8_DMA_TAIL(NTS)                                                                     \
  asm volatile(                                                                                  \
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"                                      \
      "global_load_lds_dwordx4 %1, %3 offset:2048" NTS "\n\t"                                    \
      "s_mov_b32 m0, %0"                                                                         \
      : "=&s"(sv)                                                                                \
      : "v"(voff), "s"(lds + 8192), "s"(b2)                                                      \
      : "memory")
  if constexpr (NT) {
    MLA_F8_DMA(" nt");
    if (tail_lane) MLA_F8_DMA_TAIL(" nt");
  } else {
    MLA_F8_DMA("");
    if (tail_lane) MLA_F8_DMA_TAIL("");
  }
#undef MLA_F8_DMA
#undef MLA_F8_DMA_TAIL
}

// One bf16 block into an LDS stage: 18 loads of 16 B per lane.  Load j = 4m + q reads chunk
// block j / 2 (bytes 128 (j / 2) ..) of the lane's row (vo0: its byte offset from the block's
// first row for even loads, vo1 for odd ones) and writes 1 KB at stage + 1024 j.  It is a
// global load with an SGPR base: address = base_m + voff_q + 1024 q with base_m = row0 +
// 256 m - 3072 and voff_q = vo_(q & 1) + 128 (q >> 1) - 1024 q + 3072 (>= 0), and the same
// instruction offset 1024 q lands in LDS at M0 + 1024 q with M0 = stage + 4096 m, so M0
// changes once per four loads (saved and restored around them).  Like dma_f8_block it first
// waits for the LDS reads issued before it, and it is hidden from the compiler's counters.
template <bool NT>
__device__ __forceinline__ void dma_bf16_block(const uint8_t* row0, uint32_t vo0, uint32_t vo1, uint32_t lds) {
  const uint32_t v0 = vo0 + 3072, v1 = vo1 + 2048, v2 = vo0 + 1152, v3 = vo1 + 128;
  const uint8_t* b0 = row0 - 3072;
  const uint8_t* b1 = row0 - 2816;
  const uint8_t* b2 = row0 - 2560;
  const uint8_t* b3 = row0 - 2304;
  const uint8_t* b4 = row0 - 2048;
  uint32_t sv;
#define MLA_BF16_DMA4(B, NTS)                                                                     \
  "global_load_lds_dwordx4 %1, " B NTS "\n\t"                                                     \
  "global_load_lds_dwordx4 %2, " B " offset:1024" NTS "\n\t"                                      \
  "global_load_lds_dwordx4 %3, " B " offset:2048" NTS "\n\t"                                      \
  "global_load_lds_dwordx4 %4, " B " offset:3072" NTS "\n\t"
#define MLA_BF16_DMA(NTS)                                                                         \
  asm volatile(                                                                                   \
      "s_waitcnt lgkmcnt(0)\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\ts_nop 0\n\t"               \
      MLA_BF16_DMA4("%6", NTS)                                                                    \
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"                                                   \
      MLA_BF16_DMA4("%7", NTS)                                                                    \
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"                                                   \
      MLA_BF16_DMA4("%8", NTS)                                                                    \
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"                                                   \
      MLA_BF16_DMA4("%9", NTS)                                                                    \
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"                                                   \
      "global_load_lds_dwordx4 %1, %10" NTS "\n\t"                                                \
      "global_load_lds_dwordx4 %2, %10 offset:1024" NTS "\n\t"                                    \
      "s_mov_b32 m0, %0"                                                                          \
      : "=&s"(sv)                                                                                 \
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(lds), "s"(b0), "s"(b1), "s"(b2), "s"(b3), "s"(b4) \
      : "memory", "scc")
  if constexpr (NT)
    MLA_BF16_DMA(" nt");
  else
    MLA_BF16_DMA("");
#undef MLA_BF16_DMA
#undef MLA_BF16_DMA4
}
// gfx950 LDS transpose read of 16-bit elements (the V^T operand)
__device__ __forceinline__ u32x2_t lds_tr16(LDS_AS const uint8_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)p));
}

// Log-sum-exp merge of one batch of partial results into a running (M, L, acc): with
// M' = max(M, l_u), acc and L are scaled by e^(M - M') and each partial u adds
// w_u = e^(l_u - M') times its o (and w_u to L).  Partials with l = -inf (no tokens) add
// nothing.
template <int NB = kMergeBatch>
__device__ __forceinline__ void merge_batch(const float (&l)[NB], const f32x4_t (&v)[NB], float& M, float& L,
                                            f32x4_t& acc) {
  float mb = M;
#pragma unroll
  for (int u = 0; u < NB; ++u) mb = fmaxf(mb, l[u]);
  if (mb == -INFINITY) return;
  const float f = M > -INFINITY ? __expf(M - mb) : 0.f;
  L *= f;
  acc *= f;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float w = (l[u] > -INFINITY) ? __expf(l[u] - mb) : 0.f;
    L += w;
    acc += w * v[u];
  }
  M = mb;
}

// ---- Combining split sequences in the decode launch (one launch instead of two).
// Each piece's partial result goes out with device-scope stores (write-through past the
// XCD's L2); once they have completed, the work-group adds one to a device-scope counter of
// its (sequence, row group).  The one that brings it to the number of pieces resets it and
// combines every piece's partial, read with device-scope loads, exactly as merge_kernel does.
// No cache-wide write-back or invalidate is needed: only these stores and loads touch the
// partials while the launch runs.
constexpr int kAuxDevice = 16;     // cache policy of buffer loads / stores: sc1 (device scope)

// Slots of the pieces of one sequence: piece 0 in `first`, piece j > 0 in off0 + step j -- host
// schedule (off0 = first, step 1): first + j; device schedule (off0 = 2 wf, step 2): 2 wf +
// first_inside, then 2 (wf + j).
struct Pieces {
  int32_t first, count, step, off0;
};
__device__ __forceinline__ int piece_slot(const Pieces& c, int j) { return j == 0 ? c.first : c.off0 + c.step * j; }

// Buffer resource over slot s's partial rows (R x 512 floats)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const DecodeArgs& a, int s) {
  return __builtin_amdgcn_make_buffer_rsrc(a.part_o + (int64_t)s * a.rows * kDv, (short)0, a.rows * kDv * 4, 0x00020000);
}

// Thread (r, c) of 256 combines row 16 rgroup + r, columns 32 c .. 32 c + 31 over the pieces: first
// the row's max M and sum L of e^(lse - M) from the pieces' lse, then for each 8-column group
// the weighted sum of kCombineBatch pieces at a time (32 loads in flight per thread: the
// loads are latency-bound, one work-group reads every piece), then out and lse.
constexpr int kCombineBatch = 16;
template <bool OUT_F32>
__device__ __forceinline__ void combine_rows(const DecodeArgs& a, int b, int rgroup, const Pieces cm) {
  const int R = a.rows;
  const int row = 16 * rgroup + (int)(threadIdx.x >> 4);
  const int c0 = 32 * (int)(threadIdx.x & 15);
  auto lse_of = [&](int j) {
    return __hip_atomic_load(a.part_lse + (int64_t)piece_slot(cm, j) * R + row, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  };
  // M and L over the pieces, kCombineBatch lse loads in flight at a time
  float M = -INFINITY, L = 0.f;
  for (int j0 = 0; j0 < cm.count; j0 += kCombineBatch) {
    float l[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) l[u] = j0 + u < cm.count ? lse_of(j0 + u) : -INFINITY;
    float mb = M;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) mb = fmaxf(mb, l[u]);
    if (mb == -INFINITY) continue;
    L = M > -INFINITY ? L * __expf(M - mb) : 0.f;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) L += l[u] > -INFINITY ? __expf(l[u] - mb) : 0.f;
    M = mb;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  for (int q = 0; q < 4; ++q) {                    // columns 32 c + 8 q .. + 7
    const uint32_t off = (uint32_t)(row * kDv + c0 + 8 * q) * 4u;
    f32x4_t acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    for (int j0 = 0; M > -INFINITY && j0 < cm.count; j0 += kCombineBatch) {
      f32x4_t v0[kCombineBatch], v1[kCombineBatch];
      float w[kCombineBatch];
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        const bool in = j0 + u < cm.count;
        const int sl = in ? piece_slot(cm, j0 + u) : 0;
        const __amdgpu_buffer_rsrc_t rs = partial_rsrc(a, sl);
        v0[u] = in ? __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kAuxDevice))
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
        v1[u] = in ? __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, kAuxDevice))
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const float l = in ? lse_of(j0 + u) : -INFINITY;
        w[u] = l > -INFINITY ? __expf(l - M) : 0.f;     // pieces without tokens add nothing
      }
#pragma unroll
      for (int u = 0; u < kCombineBatch; ++u) {
        acc0 += w[u] * v0[u];
        acc1 += w[u] * v1[u];
      }
    }
    acc0 *= inv;
    acc1 *= inv;
    const int64_t o = ((int64_t)b * R + row) * kDv + c0 + 8 * q;
    if (OUT_F32) {
      *(f32x4_t*)((float*)a.out + o) = acc0;
      *(f32x4_t*)((float*)a.out + o + 4) = acc1;
    } else {
      *(u32x4_t*)((uint16_t*)a.out + o) = u32x4_t{bf16x2_rne(acc0[0], acc0[1]), bf16x2_rne(acc0[2], acc0[3]),
                                                  bf16x2_rne(acc1[0], acc1[1]), bf16x2_rne(acc1[2], acc1[3])};
    }
  }
  if ((threadIdx.x & 15) == 0 && a.lse) a.lse[(int64_t)b * R + row] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// After a piece's partial is out: count it; the last piece's work-group combines.  `flag`:
// 4 bytes of LDS not in use (the caller's stages are free between pieces).
template <bool OUT_F32>
__device__ __forceinline__ void combine_if_last_t(const DecodeArgs& a, int b, int rgroup, const Pieces cm,
                                                  LDS_AS int32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this thread's device-scope stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* cnt = a.merge_cnt + (int64_t)b * a.row_groups + rgroup;
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == cm.count - 1 ? 1 : 0;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
    *flag = last;
  }
  __syncthreads();
  const bool last = *flag != 0;
  __syncthreads();
  if (last) combine_rows<OUT_F32>(a, b, rgroup, cm);
}

// Split-decode kernel: 16 query rows per work-group (R = 16 * row groups).  FP8: the cache
// rows are 656-byte fp8 rows (see kF8Row); each wave streams its blocks through three fp8
// stages and builds the MFMA operands from the codes in registers (see the FP8 loop).
// DEV: no host schedule; the work-groups cut the batch's blocks among themselves from the
// device cache_seqlens and combine split sequences in the same launch (see below).
// COMB: split sequences are combined in this launch (a.merge_cnt; see combine_if_last_t).
template <bool OUT_F32, bool FP8, bool DEV, bool COMB>
__global__ void __launch_bounds__(kThreads, 1) split_decode_kernel(DecodeArgs a) {
  // the stages while blocks stream; the four waves' states (kMergeBytes) when a piece ends
  __shared__ __attribute__((aligned(1024))) uint8_t smem[FP8 ? kSplitSmemFp8 : kSplitSmemBf16];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // MFMA column (query row) / A-operand row (token or dim)
  const int g = lane >> 4;     // lane group: k sub-range of the operands

  int worker, rgroup;
  if (a.row_groups == 1) {
    worker = blockIdx.x;
    rgroup = 0;
  } else {
    // work-groups with the same token range land on the same XCD (ids are dealt round-robin to 8 XCDs)
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    rgroup = y % a.row_groups;
    worker = (y / a.row_groups) * 8 + x;
  }
  if (worker >= a.num_workers) return;
  const int row0 = rgroup * 16;
  const int R = a.rows;
  const bool stream = a.row_groups == 1;   // KV loads: non-temporal when no other row group re-reads

  // Row-major block layout (see row_swz).  K reads: token n, chunk 4*kk + g; V^T reads:
  // token 4g + e, 8-byte piece qq of a 16-column block; DMA instruction j: token
  // 8*(j & 1) + (lane >> 3), chunk 8*(j >> 1) + ((lane & 7) ^ row_swz(token)).
  const int k_even = 128 * n + 16 * (g ^ row_swz(n));
  const int k_odd = k_even ^ 64;                               // chunk 4 + g: unit index bit 2 flips
  const int e = n >> 2, qq = n & 3;
  int v_base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v_base[i] = 128 * (4 * g + e) + 16 * ((2 * i + (qq >> 1)) ^ row_swz(4 * g + e)) + 8 * (qq & 1);
  const int ld_tok0 = lane >> 3, ld_tok1 = 8 + (lane >> 3);
  const int ld_col0 = 8 * ((lane & 7) ^ row_swz(ld_tok0)), ld_col1 = 8 * ((lane & 7) ^ row_swz(ld_tok1));

  // bf16: two DMA stages per wave; FP8: kF8Stages fp8 stages per wave
  LDS_AS uint8_t* stage0 = FP8 ? lds + wave * kF8WaveBytes : lds + (wave * kStages + 0) * kBlockBytes;
  LDS_AS uint8_t* stage1 = FP8 ? stage0 + kF8Stage : lds + (wave * kStages + 1) * kBlockBytes;
  // FP8 operand addresses within a stage.  S^T: lane (t = n, g) reads token t's codes at
  // 656t + 8g (+ 32kk), its rope chunks at 656t + 512 + 16g (+ 64) and its scales at
  // 656t + 640.  O^T: the transpose read gathers, per 16-lane group g, 8-byte rows from
  // the addresses of its lanes j = 2k + p: token 4g + (k & 3), columns 16 (k >> 2) + 8p
  // (+ 32c); lane (m, g) then holds tokens 4g..4g+3 of columns 32c + m and 32c + 16 + m.
  const int f8_k = kF8Row * n + 8 * g;
  const int f8_r = kF8Row * n + 512 + 16 * g;
  const int f8_s = kF8Row * n + 640;
  const int f8_v = kF8Row * (4 * g + ((n >> 1) & 3)) + 16 * (n >> 3) + 8 * (n & 1);
  const int f8_p = kF8Row * 4 * g + 640;
  const uint8_t* const kv8 = (const uint8_t*)a.kv;

  const CST_AS int32_t* worker_off = as_const(a.worker_off);
  const CST_AS int32_t* pieces = as_const(a.pieces);
  const CST_AS int32_t* seqlens = as_const(a.seqlens);
  const CST_AS int32_t* block_table = as_const(a.block_table);

  // one piece: tokens [tb, min(te_in, L)) of sequence b; slot -1 writes out/lse, else a partial
  auto run_piece = [&](const int b, const int tb, const int te_in, const int slot) {
    if (!DEV) check_planned_length(a, b, te_in, seqlens[b]);
    const int te = min(te_in, seqlens[b]);
    const int nblk = te > tb ? (te - tb + kBlock - 1) / kBlock : 0;
    // end of the tokens this lane's query row sees: te, or for a causal problem the
    // first L - (q_len - 1 - i) tokens of the sequence (row = i * num_heads + h)
    const int lim = a.causal ? min(te, seqlens[b] - (a.q_len - 1 - (row0 + n) / a.num_heads)) : te;
    // wave w takes blocks w, w + 4, w + 8, ... of the piece
    const int my_n = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
    auto blk_of = [&](int k) { return wave + kWaves * k; };

    // query rows as MFMA B operands (Q^T), resident in VGPRs for the piece: lane (n, g) holds
    // row n, columns 32*kk + 8*g .. +8
    bf16x8_t qf[kKSteps];
    {
      const uint16_t* qrow = a.q + ((int64_t)b * R + row0 + n) * kDqk + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    }

    float m_ref = kNegBig;   // reference max (log2 units) the p values are taken against
    float lsum = 0.f;        // this lane's share of sum_t p_t (tokens 4g..4g+3 of each block)
    f32x4_t o[kVBlocks];     // O^T: lane (n, g) holds dims 16*mb + 4*g + i of row n
#pragma unroll
    for (int mb = 0; mb < kVBlocks; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // This lane's DMA sources for the wave's k-th block (even / odd instructions); `ok` is
    // false for an out-of-range table entry (then page 0 is read, in bounds, and the block
    // is skipped).  Rows past the end of the piece re-read its last valid row.
    struct Src {
      const uint8_t* row0;    // the block's first row
      uint32_t vo[2];         // bf16: this lane's byte offsets from it for even / odd loads
    };
    auto source = [&](int k, bool& ok) -> Src {
      const int tok0 = tb + kBlock * blk_of(k);
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.page_shift, a.num_pages, b, tok0);
      ok = base >= 0;
      if (!ok) base = 0;
      const int last = te - 1 - tok0;
      Src r{};
      if constexpr (FP8) {
        r.row0 = kv8 + base * kF8Row;
      } else {
        r.row0 = (const uint8_t*)(a.kv + base * kDqk);
        r.vo[0] = (uint32_t)(min(ld_tok0, last) * kRowBytesBf16 + 2 * ld_col0);
        r.vo[1] = (uint32_t)(min(ld_tok1, last) * kRowBytesBf16 + 2 * ld_col1);
      }
      return r;
    };
    // The DMA loads of a block into a stage.  bf16: 18 instructions of 1 KB, each 128 B of 8
    // rows (chunk block j/2).  FP8: the 656 16-B units of the 16 rows in row order, 64 per
    // instruction (the 11th moves the last 16).
    auto issue = [&](const Src& src, LDS_AS uint8_t* stage) {
      if constexpr (FP8) {
        // the block's 16 rows are contiguous (a block never crosses a page); rows past the
        // end of the piece are loaded too and masked where they are used
        const uint32_t l = (uint32_t)(uintptr_t)stage;
        if (stream)
          dma_f8_block<true>(src.row0, 16u * lane, l, lane < 16);
        else
          dma_f8_block<false>(src.row0, 16u * lane, l, lane < 16);
      } else {
        const uint32_t l = (uint32_t)(uintptr_t)stage;
        if (stream)
          dma_bf16_block<true>(src.row0, src.vo[0], src.vo[1], l);
        else
          dma_bf16_block<false>(src.row0, src.vo[0], src.vo[1], l);
      }
    };
    // S^T for one block and its V^T operands: the K and V^T reads are ordinary LDS loads the
    // compiler interleaves with the S^T MFMAs; halfway through the MFMAs the stage is refilled
    // with the block after next (`ns`, if `nx`; the DMA first waits for the reads), while the
    // rest of S^T, the softmax and O^T += V^T P^T are computed.
    auto scores = [&](LDS_AS uint8_t* st, f32x4_t& sacc, u32x2_t (&vf0)[16], u32x2_t (&vf1)[16], const Src& ns,
                      bool nx) {
      u32x4_t kf[kKSteps];
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) kf[kk] = lds_ld128(st + ((kk & 1) ? k_odd : k_even) + 2048 * (kk >> 1));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        vf0[i] = lds_tr16(st + v_base[i & 3] + 2048 * (i >> 2));          // columns 0..255
        vf1[i] = lds_tr16(st + v_base[i & 3] + 8192 + 2048 * (i >> 2));   // columns 256..511
      }
      f32x4_t acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        f32x4_t& acc = (kk & 1) ? acc2 : sacc;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]), qf[kk], acc, 0, 0, 0);
        if (!DEV && kk == 8 && nx) issue(ns, st);
      }
      // (the device-scheduled variant refills after S^T: halfway, its fp32-output build would
      // need a few scratch registers)
      if (DEV && nx) issue(ns, st);
      sacc += acc2;
    };
    // O^T += V^T P^T for one block, p = exp2(s - m_ref); the running sum l takes p in fp32.
    // bf16 output: p enters the MFMA in bf16.  fp32 output: p is split into two bf16 terms,
    // p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), and both go through the MFMA, so the
    // weights carry ~16 mantissa bits instead of bf16's 8.
    auto accumulate = [&](const float (&s)[4], const u32x2_t (&vf0)[16], const u32x2_t (&vf1)[16]) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        lsum += p[i];
      }
      auto pv = [&](const u32x2_t (&vf)[16], int mb0) {
        if constexpr (OUT_F32) {
          // fp32 output: one 16x16x32 MFMA per column block, K index 8g + j being token
          // 4g + (j & 3) with p's hi part for j < 4 and its lo part for j >= 4, against V^T
          // repeated twice
          const u32x4_t pp = split_hi_lo(p[0], p[1], p[2], p[3]);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const u32x4_t v = u32x4_t{vf[i][0], vf[i][1], vf[i][0], vf[i][1]};
            o[mb0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v),
                                                                 __builtin_bit_cast(bf16x8_t, pp), o[mb0 + i], 0, 0, 0);
          }
        } else {
          // bf16 output: p in bf16, one 16x16x16 MFMA per column block (K index 4g + j is
          // token 4g + j)
          const u32x2_t pp = u32x2_t{bf16x2_rne(p[0], p[1]), bf16x2_rne(p[2], p[3])};
#pragma unroll
          for (int i = 0; i < 16; ++i)
            o[mb0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, vf[i]),
                                                                   __builtin_bit_cast(i16x4_t, pp), o[mb0 + i], 0, 0, 0);
        }
      };
      pv(vf0, 0);
      pv(vf1, 16);
    };

    // FP8: O^T += V^T P^T with V^T the codes (converted exactly to bf16, scale 1) and, for
    // the columns of group G, P^T scaled by each token's 2^e[t][G], the exponent part of its
    // group scale; p_t 2^e is split into hi + lo exactly as p is on the bf16 path.  vr holds
    // the transposed codes (4 reads per group) and psc the scales of tokens 4g..4g+3.  Rows
    // past the end of the piece were zeroed in the stage (codes and scales), so they add
    // nothing.
    auto accumulate_f8 = [&](const float (&s)[4], const u32x2_t (&vr)[16], const u32x4_t (&psc)[4]) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        lsum += p[i];
      }
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        float pg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pg[i] = p[i] * __uint_as_float(psc[i][G] & 0x7F800000u);
        // fp32 output: p 2^e as hi + lo on the K axis of a 16x16x32 MFMA (as on the bf16
        // path); bf16 output: p 2^e in bf16 on a 16x16x16 MFMA
        const u32x4_t pp = OUT_F32 ? split_hi_lo(pg[0], pg[1], pg[2], pg[3])
                                   : u32x4_t{bf16x2_rne(pg[0], pg[1]), bf16x2_rne(pg[2], pg[3]), 0u, 0u};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int c = 4 * G + cc;               // 32-column chunk (tiles 2c, 2c + 1)
          const uint32_t w0 = vr[c][0], w1 = vr[c][1];
          const uint32_t l0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
          const uint32_t l1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
          const uint32_t h0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
          const uint32_t h1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
          if constexpr (OUT_F32) {
            o[2 * c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u32x4_t{l0, l1, l0, l1}),
                                                               __builtin_bit_cast(bf16x8_t, pp), o[2 * c], 0, 0, 0);
            o[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u32x4_t{h0, h1, h0, h1}),
                                                                   __builtin_bit_cast(bf16x8_t, pp), o[2 * c + 1], 0, 0, 0);
          } else {
            const i16x4_t pb = __builtin_bit_cast(i16x4_t, u32x2_t{pp[0], pp[1]});
            o[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, u32x2_t{l0, l1}), pb,
                                                                 o[2 * c], 0, 0, 0);
            o[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, u32x2_t{h0, h1}), pb,
                                                                     o[2 * c + 1], 0, 0, 0);
          }
        }
      }
    };

    if constexpr (FP8) {
      // ---- FP8 rows: three stages per wave; block k is in stage k % 3 while blocks k + 1
      // and k + 2 are in flight.  All of block k's operands are read from the stage (the
      // compiler interleaves the reads with the S^T MFMAs), and halfway through S^T the
      // stage is refilled with block k + 3.  S^T takes K = code * scale from the conversion (which applies the
      // scale's exponent); O^T takes V^T = code and folds each token's group scale 2^e into
      // P (exact for powers of two): O^T[d] += sum_t code[t][d] (p_t 2^e[t][d/128]).
      uint32_t okq = 0;   // bit i: the table entry of the block now in stage i was in range
#pragma unroll
      for (int i = 0; i < kF8Stages; ++i) {
        bool ok = true;
        if (i < my_n) issue(source(i, ok), stage0 + i * kF8Stage);
        okq |= (ok ? 1u : 0u) << i;
      }
      int k = 0;
      while (k < my_n) {
        float s[4], mx = 0.f;
        bool rescale = false;
        u32x2_t vr[16];
        u32x4_t psc[4];
        for (; k < my_n; ++k) {
          const int slot = k % kF8Stages;
          LDS_AS uint8_t* const st = stage0 + slot * kF8Stage;
          const int after = min(kF8Stages - 1, my_n - 1 - k);   // blocks issued after block k
          if (after >= 2)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kF8Loads) : "memory");
          else if (after == 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kF8Loads) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          const bool ok = (okq >> slot) & 1u;
          // A block whose table entry was out of range (its DMA read page 0) takes the same
          // path with every row zeroed and every score masked, so it adds nothing; one loop
          // body without a skip keeps the accumulators in place across iterations.
          if (!ok && lane == 0) __hip_atomic_fetch_or(a.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int tok0 = tb + kBlock * blk_of(k);
          const int vvalid = ok ? te - tok0 : 0;    // rows of the block inside the piece
          if (vvalid < kBlock) {
            // rows vvalid..15 may hold anything: zero their codes, rope and scales in the stage
            for (int u = (kF8Row / 16) * vvalid + lane; u < kF8Units; u += 64)
              *(LDS_AS u32x4_t*)(st + 16 * u) = u32x4_t{0u, 0u, 0u, 0u};
          }
          // block k's operands
          const u32x4_t ksc = lds_ld128(st + f8_s);
          u32x2_t kr[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) kr[i] = lds_ld64(st + f8_k + 32 * i);
          const u32x4_t rope0 = lds_ld128(st + f8_r), rope1 = lds_ld128(st + f8_r + 64);
#pragma unroll
          for (int c = 0; c < 16; ++c) vr[c] = lds_tr8(st + f8_v + 32 * c);
#pragma unroll
          for (int i = 0; i < 4; ++i) psc[i] = lds_ld128(st + f8_p + kF8Row * i);
          // S^T = K Q^T: 16 k-steps from the codes, then the two rope k-steps
          f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) {
            const float sc = __uint_as_float(ksc[kk >> 2] & 0x7F800000u);   // the scale's exponent only
            u32x4_t kf;
            kf[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[kk][0], sc, false));
            kf[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[kk][0], sc, true));
            kf[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[kk][1], sc, false));
            kf[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[kk][1], sc, true));
            f32x4_t& acc = (kk & 1) ? acc2 : sacc;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[kk], acc, 0, 0, 0);
            if (kk == 8) {
              // refill the stage with block k + 3 (the DMA waits for the block's reads first)
              bool nok = true;
              if (k + kF8Stages < my_n) issue(source(k + kF8Stages, nok), st);
              okq = (okq & ~(1u << slot)) | ((nok ? 1u : 0u) << slot);
            }
          }
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, rope0), qf[16], sacc, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, rope1), qf[17], acc2, 0, 0, 0);
          sacc += acc2;
          const int nvalid = ok ? lim - tok0 : 0;   // tokens of the block this row sees (may be <= 0)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i] = (4 * g + i < nvalid) ? sacc[i] * a.scale_log2 : -INFINITY;
          mx = wave_max_over_groups(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
          if (__any(mx > m_ref + kRescaleSlack)) {
            rescale = true;
            break;
          }
          accumulate_f8(s, vr, psc);
        }
        if (!rescale) break;
        {
          // rare path: a running max grew past the slack; move the reference and rescale
          // (block k's operands are still in vr and psc)
          const bool need = mx > m_ref + kRescaleSlack;
          const float f = need ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
          m_ref = need ? mx : m_ref;
          lsum *= f;
#pragma unroll
          for (int mb = 0; mb < kVBlocks; ++mb) o[mb] *= f;
          accumulate_f8(s, vr, psc);
          ++k;
        }
      }
    } else {
    bool ok0 = true, ok1 = true;   // table entry of the block now in each stage was in range
      if (my_n > 0) issue(source(0, ok0), stage0);
      if (my_n > 1) issue(source(1, ok1), stage1);

      int k = 0;
      while (k < my_n) {
        float s[4], mx = 0.f;
        bool rescale = false;
        u32x2_t vf0[16], vf1[16];
        // hot loop: o is only touched by MFMA here
        for (; k < my_n; ++k) {
          LDS_AS uint8_t* st = (k & 1) ? stage1 : stage0;
          bool nok = true;
          const bool nx = k + 2 < my_n;
          Src nsrc{};
          if (nx) nsrc = source(k + 2, nok);
          if (k + 1 < my_n) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerBlock) : "memory");
          } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          }
          const bool ok = (k & 1) ? ok1 : ok0;
          if (k & 1) ok1 = nok; else ok0 = nok;   // the stage's next occupant
          if (!ok) {
            if (lane == 0) __hip_atomic_fetch_or(a.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (nx) issue(nsrc, st);
            continue;
          }
          const int tok0 = tb + kBlock * blk_of(k);
          f32x4_t sacc;
          scores(st, sacc, vf0, vf1, nsrc, nx);
          const int nvalid = lim - tok0;   // tokens of the block this row sees (may be <= 0)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i] = (4 * g + i < nvalid) ? sacc[i] * a.scale_log2 : -INFINITY;
          mx = wave_max_over_groups(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
          if (__any(mx > m_ref + kRescaleSlack)) {
            rescale = true;
            break;
          }
          accumulate(s, vf0, vf1);
        }
        if (!rescale) break;
        // rare path: a running max grew past the slack; move the reference and rescale
        {
          const bool need = mx > m_ref + kRescaleSlack;
          const float f = need ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
          m_ref = need ? mx : m_ref;
          lsum *= f;
#pragma unroll
          for (int mb = 0; mb < kVBlocks; ++mb) o[mb] *= f;
          accumulate(s, vf0, vf1);
          ++k;
        }
      }

    }

    // ---- merge the four waves' states and write
    {
      const float lrow = wave_sum_over_groups(lsum);
      __syncthreads();   // stages no longer read
      LDS_AS float* buf = (LDS_AS float*)smem;                     // [4 waves][16 rows][516]
      LDS_AS float* sm_m = buf + kWaves * 16 * kMergeStride;       // [4][16]
      LDS_AS float* sm_l = sm_m + kWaves * 16;                     // [4][16]
      if (g == 0) {
        sm_m[wave * 16 + n] = m_ref;
        sm_l[wave * 16 + n] = lrow;
      }
      {
        LDS_AS float* my = buf + (wave * 16 + n) * kMergeStride + 4 * g;
#pragma unroll
        for (int mb = 0; mb < kVBlocks; ++mb) *(LDS_AS f32x4_t*)(my + 16 * mb) = o[mb];
      }
      __syncthreads();
      const int r = threadIdx.x >> 4, dseg = threadIdx.x & 15;
      float mw[kWaves], M = kNegBig;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = sm_m[w * 16 + r];
        M = fmaxf(M, mw[w]);
      }
      float fw[kWaves], L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        fw[w] = (mw[w] <= kNegBig) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        L += fw[w] * sm_l[w * 16 + r];
      }
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      const int grow = row0 + r;
#pragma unroll
      for (int j = 0; j < kDv / 64; ++j) {
        const int d = 4 * dseg + 64 * j;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += fw[w] * *(LDS_AS const f32x4_t*)(buf + (w * 16 + r) * kMergeStride + d);
        acc *= inv;
        if (slot < 0) {
          const int64_t off = ((int64_t)b * R + grow) * kDv + d;
          if (OUT_F32) {
            *(f32x4_t*)((float*)a.out + off) = acc;
          } else {
            u32x2_t pkd;
            pkd[0] = bf16x2_rne(acc[0], acc[1]);
            pkd[1] = bf16x2_rne(acc[2], acc[3]);
            *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
          }
        } else if constexpr (COMB) {
          // device-scope (write-through) store: read back by another work-group in this launch
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc), partial_rsrc(a, slot),
                                                 (uint32_t)(grow * kDv + d) * 4u, 0, kAuxDevice);
        } else {
          *(f32x4_t*)(a.part_o + ((int64_t)slot * R + grow) * kDv + d) = acc;
        }
      }
      if (dseg == 0) {
        const float lse = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
        if (slot < 0) {
          if (a.lse) a.lse[(int64_t)b * R + grow] = lse;
        } else if constexpr (COMB) {
          __hip_atomic_store(a.part_lse + (int64_t)slot * R + grow, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          a.part_lse[(int64_t)slot * R + grow] = lse;
        }
      }
    }
    __syncthreads();
  };

  if constexpr (!DEV) {
    // the worker's piece range is read together with the plan id (both lie inside the workspace
    // whatever schedule it holds); the pieces themselves only once the id matches
    const int p_begin = worker_off[worker], p_end = worker_off[worker + 1];
    if (!schedule_matches(a)) return;
    for (int pi = p_begin; pi < p_end; ++pi)
    {
      const int b = pieces[4 * pi + 0], slot = pieces[4 * pi + 3];
      run_piece(b, pieces[4 * pi + 1], pieces[4 * pi + 2], slot);
      // combined in this launch: the sequence's slots are seq_merge[b][0] + 0 .. count - 1
      if (COMB && slot >= 0) {
        const int first = a.seq_merge[2 * b];
        combine_if_last_t<OUT_F32>(a, b, rgroup, Pieces{first, a.seq_merge[2 * b + 1], 1, first},
                                   (LDS_AS int32_t*)smem);
      }
    }
    return;
  } else {
    // ---- device schedule.  The batch's 16-token blocks, sequence after sequence, form
    // one range [0, T); with W = min(num_workers, T / kMinBlocks) (at least 1), work-group
    // w < W takes blocks [floor(wT/W), floor((w+1)T/W)) and cuts them at sequence
    // boundaries.  A sequence met by several work-groups is split: its piece in work-group
    // w writes partial slot 2w (when the sequence began before w's range) or 2w + 1 (when
    // it begins inside it, so at most one piece per slot), and merge_dev_kernel combines
    // them in the next launch from the cut each sequence's first piece records.
    const int B = a.batch;
    const int cap = a.bt_stride * a.page_size;            // tokens one block-table row maps
    auto seq_len = [&](int bb) { return max(0, min(seqlens[bb], cap)); };
    auto seq_blocks = [&](int bb) { return (seq_len(bb) + kBlock - 1) / kBlock; };
    // block prefix over the batch: each thread sums a contiguous chunk, then an inclusive
    // scan of the 256 chunk sums (the LDS stages are not in use yet)
    LDS_AS int32_t* sums = (LDS_AS int32_t*)smem;         // [2][256]
    const int per = (B + kThreads - 1) / kThreads;
    const int c0 = min(B, (int)threadIdx.x * per), c1 = min(B, c0 + per);
    int mine = 0;
    for (int bb = c0; bb < c1; ++bb) mine += (max(0, min(a.seqlens[bb], cap)) + kBlock - 1) / kBlock;
    sums[threadIdx.x] = mine;
    __syncthreads();
    int src = 0;
    for (int d = 1; d < kThreads; d <<= 1) {
      const int v = sums[src * kThreads + threadIdx.x] +
                    ((int)threadIdx.x >= d ? sums[src * kThreads + threadIdx.x - d] : 0);
      sums[(src ^ 1) * kThreads + threadIdx.x] = v;
      __syncthreads();
      src ^= 1;
    }
    const int64_t T = sums[src * kThreads + kThreads - 1];
    // at least kMinBlocks blocks per work-group (one per wave): short batches use fewer
    const int W = (int)max<int64_t>(1, min<int64_t>(a.num_workers, T / kMinBlocks));
    const int64_t s0 = worker < W ? T * worker / W : T, e0 = worker < W ? T * (worker + 1) / W : T;
    // the chunk holding block s0, then the sequence in it (uniform: every lane computes it)
    int ch = 0;
    for (int lo = 0, hi = kThreads - 1; lo < hi;) {
      const int mid = (lo + hi) >> 1;
      if (sums[src * kThreads + mid] > s0) hi = mid; else lo = mid + 1;
      ch = lo;
    }
    int64_t pre = ch > 0 ? sums[src * kThreads + ch - 1] : 0;   // blocks before chunk ch
    __syncthreads();                                       // the stages may overwrite sums now
    int bcur = min(B, ch * per);
    while (bcur < B && pre + seq_blocks(bcur) <= s0) pre += seq_blocks(bcur++);
    // worker holding block x of the range (the largest w with floor(wT/W) <= x)
    auto wpos = [&](int64_t x) { return (int)(((x + 1) * W - 1) / T); };
    auto wstart = [&](int w) { return T * w / W; };
    for (; bcur < B && pre < e0; pre += seq_blocks(bcur++)) {
      const int64_t p0 = pre, p1 = pre + seq_blocks(bcur);
      if (p1 == p0) continue;                              // empty: handled below
      const int64_t lo = max(p0, s0), hi = min(p1, e0);
      const bool split = p0 < s0 || p1 > e0;
      const int slot = split ? 2 * worker + (p0 > s0 ? 1 : 0) : -1;
      if (lo == p0 && rgroup == 0 && threadIdx.x == 0) {
        // the sequence's first piece records how it was cut, for the merge launch
        const int wf = wpos(p0), wl = wpos(p1 - 1);
        int4 info = {split ? wf : -1, wl, p0 > wstart(wf) ? 1 : 0, 0};
        *(int4*)(a.seq_info + 4 * bcur) = info;
      }
      run_piece(bcur, (int)(lo - p0) * kBlock, (int)(hi - p0) * kBlock, slot);
      if (COMB && slot >= 0) {
        // the pieces of the sequence: work-groups wf..wl, slots 2w (2 wf + 1 when it begins inside wf's range)
        const int wf = wpos(p0), wl = wpos(p1 - 1);
        combine_if_last_t<OUT_F32>(a, bcur, rgroup, Pieces{2 * wf + (p0 > wstart(wf) ? 1 : 0), wl - wf + 1, 2, 2 * wf},
                                   (LDS_AS int32_t*)smem);
      }
    }
    if (worker == 0 && rgroup == 0 && threadIdx.x == 0) {
      a.seq_info[4 * B + 0] = (int32_t)T;                 // schedule header: T and W
      a.seq_info[4 * B + 1] = W;
    }
    // empty sequences: work-group w < W writes those with index = w (mod W)
    for (int bb = worker; worker < W && bb < B; bb += W) {
      if (seq_blocks(bb) != 0) continue;
      if (rgroup == 0 && threadIdx.x == 0) *(int4*)(a.seq_info + 4 * bb) = int4{-1, -1, 0, 0};
      const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
      const int64_t off = ((int64_t)bb * R + row0 + r) * kDv + 32 * c;
      for (int i = 0; i < 32; ++i) {
        if (OUT_F32) ((float*)a.out)[off + i] = 0.f;
        else ((uint16_t*)a.out)[off + i] = 0;
      }
      if (c == 0 && a.lse) a.lse[(int64_t)bb * R + row0 + r] = -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Wide split-decode kernel: 128 query rows per work-group, 32 per wave, on 32x32x16 bf16 MFMA
// (or 64 rows, each set of 32 shared by two waves that split the output columns; see CW below).
//
// The four waves consume every 32-token block of a piece from a shared ring of four LDS slots
// (three blocks in flight while one is computed); wave w moves token octet w of each block
// (9 global->LDS loads of 1 KB).  Wave w owns query rows 32w..32w+31 of the row group:
//   S^T = K Q^T     M = 32 tokens, N = 32 rows, K = 576 (36 MFMAs); Q^T's 512 latent columns
//                   resident in VGPRs, its 64 rope columns in the LDS left beside the slots
//   P^T = exp2(S^T - m)                                   (16 scores per lane)
//   O^T += V^T P^T  M = 32 columns, N = 32 rows, K = 16 tokens (2 MFMAs per 32-column tile)
// so every K and V^T byte read from LDS feeds 32 query rows (the transposed flow of the
// FlashMLA-ETAP summary, "Core mechanism", with the matrix unit's wide 32x32 shape filled by
// tokens and rows alike).  O^T (512 x 32 per wave) stays in accumulation registers.
//
// Softmax without mid-stream rescaling: each row's reference m is the maximum of its scores in
// the piece's first block, and p = exp2(s - m) is accumulated as is while every later score
// stays within kWSlack (log2 units) of m (p <= 2^32: no overflow in bf16 or fp32).  A piece in
// which some score exceeds that is computed once more from the start with m set to the row's
// true maximum, which the first pass has found; so the accumulators are only ever touched by
// MFMAs.
//
// Block layout in LDS (16-B units): chunk c (columns 8c..8c+7) of token t sits at unit
// 256 (c / 8) + 8 t + ((c % 8) ^ wswz(t)).  One DMA load fills 8 tokens x 8 chunks; the swizzle
// makes the K reads (32 tokens x one chunk) and the V^T transpose reads (4 tokens x 16 columns
// per 16 lanes) hit distinct banks.
constexpr int kWBlock = 32;                              // tokens per block
constexpr int kWBlockBytes = kWBlock * kRowBytesBf16;    // 36,864
constexpr int kWSlots = 4;
constexpr int kWQRope = kWSlots * kWBlockBytes;          // the query's rope columns: [wave][4][64 lanes] x 16 B
constexpr int kWSmem = kWQRope + kWaves * 4 * 64 * 16;   // 163,840: all of the LDS
constexpr float kWSlack = 32.0f;
constexpr int kWRing = 4;                                // K operands in flight in S^T
constexpr int kWVRing = 3;                               // V^T operands (32-column tiles) in flight in O^T

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int wswz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
// byte offset of chunk c of token t within a block
__device__ __forceinline__ int wunit(int t, int c) { return 16 * (256 * (c >> 3) + 8 * t + ((c & 7) ^ wswz(t))); }

// One wave's token octet of a block: load cg (0..8) reads 16 B per lane at base + voff + 128 cg
// and writes 1 KB at m0 + 4096 cg (the instruction offset applies to both addresses, so M0
// steps by 3,968).  Saves and restores M0; hidden from the compiler's counters.
template <bool NT>
__device__ __forceinline__ void dma_wide_octet(const uint8_t* base, uint32_t voff, uint32_t m0) {
  uint32_t sv;
#define MLA_W1(OFF, NTS) "s_add_u32 m0, m0, 3968\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3 offset:" OFF NTS "\n\t"
#define MLA_WIDE_DMA(NTS)                                                                       \
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"                          \
               "global_load_lds_dwordx4 %1, %3" NTS "\n\t"                                    \
               MLA_W1("128", NTS) MLA_W1("256", NTS) MLA_W1("384", NTS) MLA_W1("512", NTS)    \
               MLA_W1("640", NTS) MLA_W1("768", NTS) MLA_W1("896", NTS) MLA_W1("1024", NTS)   \
               "s_mov_b32 m0, %0"                                                             \
               : "=&s"(sv)                                                                    \
               : "v"(voff), "s"(m0), "s"(base)                                                \
               : "memory", "scc")
  if constexpr (NT)
    MLA_WIDE_DMA(" nt");
  else
    MLA_WIDE_DMA("");
#undef MLA_WIDE_DMA
#undef MLA_W1
}

// One global->LDS load of 1 KB: 16 B per lane from base + voff + OFF into LDS at m0 + OFF + 16 lane
// (the instruction offset applies to both addresses).  Saves and restores M0; hidden from the
// compiler's counters.
template <bool NT, int OFF>
__device__ __forceinline__ void dma_one(const uint8_t* base, uint32_t voff, uint32_t m0) {
  uint32_t sv;
  if constexpr (NT)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3 offset:%4 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(sv)
                 : "v"(voff), "s"(m0), "s"(base), "n"(OFF)
                 : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3 offset:%4\n\ts_mov_b32 m0, %0"
                 : "=&s"(sv)
                 : "v"(voff), "s"(m0), "s"(base), "n"(OFF)
                 : "memory");
}

// FP8 rows in the wide kernel: one wave's token octet of a block as 6 loads of 1 KB.  Each lane
// gathers 16-B units so that the wave's own 1 KB areas of the slot (at m0 + 4096 region) hold
//   regions 1, 3, 5, 7: code pair j (columns 128 j .. 128 j + 127 of the 8 tokens: lane 8 r + y
//                       loads bytes 128 j + 16 y of token r; vcode = row + 16 y, offset 128 j),
//   region 6:           the four group scales of token L / 8 at 16 L (every lane of a token
//                       loads the same 16 B),
//   region 8:           the bf16 rope chunks, already in the bf16 layout (vrope as the bf16 DMA).
// The wave then converts the codes in place (wide_decode_kernel, `convert`) into regions 0..7.
// Offsets stay below 4096, so M0 steps per load: 4096, then +8064 three times (region 2 j + 1
// minus the instruction offset 128 j), -3712 to region 6, +8192 to region 8.
template <bool NT>
__device__ __forceinline__ void dma_wide_f8(const uint8_t* base, uint32_t vcode, uint32_t vscale, uint32_t vrope,
                                            uint32_t m0) {
  uint32_t sv;
#define MLA_WF8(NTS)                                                                              \
  asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %4, 4096\n\ts_nop 0\n\t"                   \
               "global_load_lds_dwordx4 %1, %5" NTS "\n\t"                                     \
               "s_add_u32 m0, m0, 8064\n\ts_nop 0\n\t"                                          \
               "global_load_lds_dwordx4 %1, %5 offset:128" NTS "\n\t"                          \
               "s_add_u32 m0, m0, 8064\n\ts_nop 0\n\t"                                          \
               "global_load_lds_dwordx4 %1, %5 offset:256" NTS "\n\t"                          \
               "s_add_u32 m0, m0, 8064\n\ts_nop 0\n\t"                                          \
               "global_load_lds_dwordx4 %1, %5 offset:384" NTS "\n\t"                          \
               "s_sub_u32 m0, m0, 3712\n\ts_nop 0\n\t"                                          \
               "global_load_lds_dwordx4 %2, %5" NTS "\n\t"                                     \
               "s_add_u32 m0, m0, 8192\n\ts_nop 0\n\t"                                          \
               "global_load_lds_dwordx4 %3, %5" NTS "\n\t"                                     \
               "s_mov_b32 m0, %0"                                                              \
               : "=&s"(sv)                                                                     \
               : "v"(vcode), "v"(vscale), "v"(vrope), "s"(m0), "s"(base)                       \
               : "memory", "scc")
  if constexpr (NT)
    MLA_WF8(" nt");
  else
    MLA_WF8("");
#undef MLA_WF8
}
constexpr int kWF8Loads = 6;
// Block k + 2's loads are spread over block k's 36 S^T steps (issued together, right after the
// barrier, the four waves' loads queue behind each other): load j at step kWDma0 + kWDmaStride j.
constexpr int kWDma0 = 1, kWDmaStride = 4;                 // bf16: 9 loads, steps 1 .. 33
constexpr int kWDma0F8 = 4, kWDmaStrideF8 = 6;             // FP8: 6 loads, steps 4 .. 34
static_assert(kWDma0 + 8 * kWDmaStride < 36 && kWDma0F8 + 5 * kWDmaStrideF8 < 36, "load steps");
// Where the conversion of the next block sits among the S^T steps: its loads are waited for at
// step kWCvWait (before any of block k + 2's loads is issued, so that the wait is for all loads
// in flight), code pair j is read at step kWCvWait + 1 + kWCvStride j and written kWCvLag steps
// later.
constexpr int kWCvWait = 2;
constexpr int kWCvStride = 6;
constexpr int kWCvLag = 4;
static_assert(kWCvWait + 1 + 3 * kWCvStride + kWCvLag < 36 && kWCvLag <= kWCvStride && kWCvWait < kWDma0F8,
              "conversion steps");

// S^T steps on a 32x32x16 bf16 MFMA with the accumulator in VGPRs: the 512 x 32 O^T tile fills
// all 256 accumulation registers, and the builtin would borrow 16 of them (moving an O^T tile out
// and back around every block).  acc = a b (first step, no accumulator input), acc += a b, and the
// last step, which adds 20 wait states so that vector instructions may read acc right after it
// (an 8-pass MFMA result read by the VALU needs 11; back-to-back accumulation into the same
// registers needs none).
__device__ __forceinline__ void mfma32_vfirst(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vacc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vlast(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc) : "v"(a), "v"(b));
}

template <bool OUT_F32, bool NT, bool FP8, int CW>
__global__ void __launch_bounds__(kThreads, 1) wide_decode_kernel(DecodeArgs a) {
  constexpr int kRowB = FP8 ? kF8Row : kRowBytesBf16;    // bytes per cache row
  // CW waves share each set of 32 rows, each computing the rows' S^T and its own NC of the 16
  // 32-column O^T tiles: 128 rows per work-group (CW = 1) or 64 (CW = 2).  (With 32 rows, four
  // waves repeating S^T cost more than the 32-row kernel's split of the tokens.)
  static_assert(CW == 1 || CW == 2, "waves per 32 rows");
  constexpr int NC = 16 / CW;                 // O^T tiles per wave
  constexpr int RW = kWaves / CW;             // 32-row sets per work-group
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWSmem];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, h = lane >> 5;

  int worker, rgroup;
  if (a.row_groups == 1) {
    worker = blockIdx.x;
    rgroup = 0;
  } else {
    // the row groups of one token range land on the same XCD (ids are dealt round-robin to 8 XCDs)
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    rgroup = y % a.row_groups;
    worker = (y / a.row_groups) * 8 + x;
  }
  if (worker >= a.num_workers) return;
  const int R = a.rows;
  const int rbase = rgroup * (32 * RW) + 32 * (wave / CW);
  const int row = rbase + i;
  const int tile0 = NC * (wave % CW);         // this wave's first O^T tile (32 columns each)
  LDS_AS uint8_t* const qrope = lds + kWQRope + 4096 * wave + 16 * lane;   // this lane's rope operands

  // LDS read offsets within a block.  K, k-step kk: token i, chunk 2 kk + h, at
  // kb0 ^ 32 (kk % 4) + 4096 (kk / 4) (chunk bits 1-2 sit at byte bits 5-6, above the xor's reach)
  const int kb0 = wunit(i, h);
  // V^T, 32-column tile cc, token half u, part jp: lane n = 4e + qq of 16-lane group g addresses
  // token 16u + 8jp + 4(g / 2) + e, the 8 bytes of columns 32cc + 16(g % 2) + 4qq..+3; the
  // transpose hands lane (i, h) column 32cc + i of tokens 16u + 8jp + 4h + 0..3.
  //   offset = (vb[jp] ^ 64 (cc % 2)) + 4096 (cc / 2) + 2048 u  (an odd tile flips chunk bit 2, byte bit 6)
  int vb[2];
  {
    const int g = lane >> 4, n = lane & 15, e = n >> 2, qq = n & 3;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) vb[jp] = wunit(8 * jp + 4 * (g >> 1) + e, 2 * (g & 1) + (qq >> 1)) + 8 * (qq & 1);
  }
  // DMA: lane L moves token 8 wave + L / 8 of the block, chunks 8 cg + ((L % 8) ^ wswz(token))
  const int dma_tok = 8 * wave + (lane >> 3);
  const uint32_t dma_col = 16u * (uint32_t)((lane & 7) ^ wswz(dma_tok));
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // FP8 conversion (lane L = 8 r + x converts token r of the wave's octet): the bf16 unit it
  // writes at 1024 wave + 16 L of region cg holds chunk c = 8 cg + xs, xs = x ^ wswz(token), i.e.
  // codes 8 c .. 8 c + 7, which code pair cg / 2 holds at unit 8 r + 4 (cg % 2) + xs / 2, half xs % 2
  const int cv_xs = (lane & 7) ^ wswz(dma_tok);
  const int cv_rd = 1024 * wave + 16 * (8 * (lane >> 3) + (cv_xs >> 1)) + 8 * (cv_xs & 1);
  const int cv_wr = 1024 * wave + 16 * lane;

  const CST_AS int32_t* worker_off = as_const(a.worker_off);
  const CST_AS int32_t* pieces = as_const(a.pieces);
  const CST_AS int32_t* seqlens = as_const(a.seqlens);
  const CST_AS int32_t* block_table = as_const(a.block_table);
  const uint8_t* const kv8 = (const uint8_t*)a.kv;

  // the piece range is read with the plan id, the pieces once the id matches
  const int p_begin = worker_off[worker], p_end = worker_off[worker + 1];
  if (!schedule_matches(a)) return;
  for (int pi = p_begin; pi < p_end; ++pi) {
    const int b = pieces[4 * pi + 0];
    const int tb = pieces[4 * pi + 1];
    check_planned_length(a, b, pieces[4 * pi + 2], seqlens[b]);
    const int L = seqlens[b];
    const int te = min(pieces[4 * pi + 2], L);
    const int slot = pieces[4 * pi + 3];
    const int nblk = te > tb ? (te - tb + kWBlock - 1) / kWBlock : 0;
    // end of the tokens this lane's row sees (causal: the first L - (q_len - 1 - i)); the
    // smallest over the wave's rows is its first row's (rows increase with the query token)
    const int lim = a.causal ? min(te, L - (a.q_len - 1 - row / a.num_heads)) : te;
    const int lim_min = a.causal ? min(te, L - (a.q_len - 1 - rbase / a.num_heads)) : te;

    // query rows as MFMA B operands: lane (i, h) holds row i, columns 16 kk + 8 h .. + 7; the
    // latent k-steps (kk < 32) in VGPRs, the rope ones in this lane's LDS area (only this wave
    // reads it, in program order after the writes)
    bf16x8_t qf[32];
    {
      // the wave's first row (uniform) plus a 32-bit lane offset
      const uint8_t* qw = (const uint8_t*)(a.q + ((int64_t)b * R + rbase) * kDqk);
      const uint32_t qo = (uint32_t)i * kRowBytesBf16 + 16u * h;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) qf[kk] = *(const bf16x8_t*)(qw + qo + 32 * kk);
#pragma unroll
      for (int kr = 0; kr < 4; ++kr) *(LDS_AS u32x4_t*)(qrope + 1024 * kr) = *(const u32x4_t*)(qw + qo + 1024 + 32 * kr);
      // every query load has landed (an s_waitcnt the compiler sees, so that it does not wait
      // for them again inside the block loop, where its count would include the DMA loads)
      __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    }

    // Block k's page walk: the table entries (physical pages) of its two 16-token halves'
    // first tokens (clamped to the piece) and those tokens' rows within their pages.  A half
    // never spans two pages (pieces start on 16-token boundaries and pages hold a multiple of 16
    // tokens).  walk() only reads the two entries, with no branch or use between the reads, so
    // that both are in flight together; publish() uses them after its barrier, so that they are
    // in flight across its waits.  An entry outside [0, num_pages) marks its half out of range.
    struct Walk {
      int g[2];      // table entries
      int off[2];    // rows within the page
    };
    const CST_AS int32_t* const bt_row = block_table + (int64_t)b * a.bt_stride;
    auto walk = [&](int k) -> Walk {
      const int t0 = tb + kWBlock * k;
      const int t1 = min(t0 + 16, te - 1);
      int p0, p1;
      if (a.page_shift >= 0) {
        p0 = t0 >> a.page_shift;
        p1 = t1 >> a.page_shift;
      } else {
        p0 = t0 / a.page_size;
        p1 = t1 / a.page_size;
      }
      return Walk{{bt_row[p0], bt_row[p1]}, {t0 - p0 * a.page_size, t1 - p1 * a.page_size}};
    };
    auto in_range = [&](int g) -> bool { return (uint32_t)g < (uint32_t)a.num_pages; };
    auto halves_ok = [&](const Walk& w) -> uint32_t { return (in_range(w.g[0]) ? 1u : 0u) | (in_range(w.g[1]) ? 2u : 0u); };
    // This wave's octet of block k (half wave / 2, 8 (wave % 2) tokens into it): its SGPR row
    // base, page 0 for an out-of-range entry (the octet is then zeroed and masked).  Lanes past
    // the end re-read the last row of the piece.
    auto octet_base = [&](int k, const Walk& w) -> const uint8_t* {
      const int g = (wave >> 1) ? w.g[1] : w.g[0];
      const int off = (wave >> 1) ? w.off[1] : w.off[0];
      const int t_half = min(tb + kWBlock * k + 16 * (wave >> 1), te - 1);     // the half's first row
      const int ts = min(tb + kWBlock * k + 8 * wave, te - 1);                  // the octet's first row
      return kv8 + (in_range(g) ? (int64_t)g * a.page_size + off + (ts - t_half) : 0) * kRowB;
    };
    auto octet_voff = [&](int k) -> uint32_t {
      const int tok0 = tb + kWBlock * k;
      const int ts = min(tok0 + 8 * wave, te - 1);
      const int t = min(tok0 + dma_tok, te - 1);
      return (uint32_t)(t - ts) * kRowB + dma_col;
    };
    // NT: non-temporal loads (one row group: no other work-group re-reads these rows)
    auto issue = [&](int k, const uint8_t* base) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((k % kWSlots) * kWBlockBytes + 1024 * wave));
      if constexpr (FP8) {
        // the row of this lane's token (its rope offset is the bf16 DMA's column offset + 512)
        const uint32_t rv = octet_voff(k) - dma_col;
        dma_wide_f8<NT>(base, rv + 16u * (uint32_t)(lane & 7), rv + 640u, rv + 512u + dma_col, m0);
      } else {
        dma_wide_octet<NT>(base, octet_voff(k), m0);
      }
    };
    // The same loads one at a time (block k + 2's, spread over block k's S^T): `pend` holds the
    // block's addresses from publish() on; part j is load j of dma_wide_octet / dma_wide_f8.
    struct Pending {
      const uint8_t* base;
      uint32_t v[3];
      uint32_t m0;
    };
    Pending pend{nullptr, {0u, 0u, 0u}, 0u};
    auto plan_issue = [&](int k, const uint8_t* base) {
      pend.base = base;
      pend.m0 = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((k % kWSlots) * kWBlockBytes + 1024 * wave));
      if constexpr (FP8) {
        const uint32_t rv = octet_voff(k) - dma_col;
        pend.v[0] = rv + 16u * (uint32_t)(lane & 7);
        pend.v[1] = rv + 640u;
        pend.v[2] = rv + 512u + dma_col;
      } else {
        pend.v[0] = octet_voff(k);
      }
    };
    auto issue_part = [&](int j) {
      if constexpr (FP8) {
        switch (j) {
          case 0: dma_one<NT, 0>(pend.base, pend.v[0], pend.m0 + 4096u); break;
          case 1: dma_one<NT, 128>(pend.base, pend.v[0], pend.m0 + 12160u); break;
          case 2: dma_one<NT, 256>(pend.base, pend.v[0], pend.m0 + 20224u); break;
          case 3: dma_one<NT, 384>(pend.base, pend.v[0], pend.m0 + 28288u); break;
          case 4: dma_one<NT, 0>(pend.base, pend.v[1], pend.m0 + 24576u); break;
          default: dma_one<NT, 0>(pend.base, pend.v[2], pend.m0 + 32768u); break;
        }
      } else {
        switch (j) {
          case 0: dma_one<NT, 0>(pend.base, pend.v[0], pend.m0); break;
          case 1: dma_one<NT, 128>(pend.base, pend.v[0], pend.m0 + 3968u); break;
          case 2: dma_one<NT, 256>(pend.base, pend.v[0], pend.m0 + 2u * 3968u); break;
          case 3: dma_one<NT, 384>(pend.base, pend.v[0], pend.m0 + 3u * 3968u); break;
          case 4: dma_one<NT, 512>(pend.base, pend.v[0], pend.m0 + 4u * 3968u); break;
          case 5: dma_one<NT, 640>(pend.base, pend.v[0], pend.m0 + 5u * 3968u); break;
          case 6: dma_one<NT, 768>(pend.base, pend.v[0], pend.m0 + 6u * 3968u); break;
          case 7: dma_one<NT, 896>(pend.base, pend.v[0], pend.m0 + 7u * 3968u); break;
          default: dma_one<NT, 1024>(pend.base, pend.v[0], pend.m0 + 8u * 3968u); break;
        }
      }
    };
    // FP8: convert this wave's octet of block k (its loads have landed) in place into the bf16
    // layout.  Code pair j becomes regions 2 j and 2 j + 1, with the group scale's exponent
    // applied by the conversion (code * 2^e is exact in bf16); an out-of-range table entry
    // (`ok` false: page 0 was read) gives zeros, rope included.  In three parts so that the
    // caller can spread them over its MFMAs: scales, then per pair the reads and the writes
    // (the writes of pair j overwrite only pairs already read, and the scales only at j = 3,
    // after the data they depend on).
    auto cv_scales = [&](int k) -> u32x4_t {
      return lds_ld128(lds + (k % kWSlots) * kWBlockBytes + 24576 + cv_wr);
    };
    auto cv_read = [&](int k, int j) -> u32x4_t {
      LDS_AS const uint8_t* st = lds + (k % kWSlots) * kWBlockBytes + 4096 * (2 * j + 1) + cv_rd;
      const u32x2_t a0 = lds_ld64(st), a1 = lds_ld64(st + 64);
      return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    };
    auto cv_write = [&](int k, int j, const u32x4_t& raw, const u32x4_t& scl, bool ok) {
      LDS_AS uint8_t* st = lds + (k % kWSlots) * kWBlockBytes + cv_wr;
      const float sc = __uint_as_float(scl[j] & 0x7F800000u);
      u32x4_t w[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          w[hh][2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2 * hh + d], sc, false));
          w[hh][2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2 * hh + d], sc, true));
        }
      *(LDS_AS u32x4_t*)(st + 4096 * (2 * j)) = w[0];
      *(LDS_AS u32x4_t*)(st + 4096 * (2 * j + 1)) = w[1];
      if (!ok) {
        // out of range (rare; ok is uniform): the same units again, zeroed (LDS writes of one
        // wave land in order), and the rope with the last pair
        *(LDS_AS u32x4_t*)(st + 4096 * (2 * j)) = u32x4_t{0u, 0u, 0u, 0u};
        *(LDS_AS u32x4_t*)(st + 4096 * (2 * j + 1)) = u32x4_t{0u, 0u, 0u, 0u};
        if (j == 3) *(LDS_AS u32x4_t*)(st + 32768) = u32x4_t{0u, 0u, 0u, 0u};
      }
    };

    float m_run = -INFINITY;     // the row's largest scaled score so far (log2 units)
    bool bad_page = false;       // an octet of this wave read an out-of-range table entry
    // scale * log2(e), kept away from zero (|c| >= 2^-100: with a smaller scale every weight
    // is 1 in float32 either way), so that the masked-token score s_hide scales to -inf
    const float c_log2 = fabsf(a.scale_log2) >= 0x1p-100f ? a.scale_log2 : copysignf(0x1p-100f, a.scale_log2);
    const float s_hide = c_log2 > 0.f ? -INFINITY : INFINITY;
    f32x16_t o[NC];
    float m_ref, lsum;
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[c][q] = 0.f;
      m_ref = pass ? fmaxf(m_run, kNegBig) : kNegBig;
      lsum = 0.f;
      bool ovf = false;
      uint32_t okq = 0;          // bits 2 (k % 4) + 0..1: block k's halves were in range
      // Blocks 0 and 1 go out first; block k + 2 is issued once block k is published.  Block
      // k's O^T update runs in iteration k + 1, interleaved with block k + 1's softmax, so the
      // slots hold: block k - 1 (its V^T being read), block k (S^T), blocks k + 1 and k + 2
      // (in flight).
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (k < nblk) {
          const Walk w = walk(k);
          issue(k, octet_base(k, w));
          okq |= halves_ok(w) << (2 * k);
        }
      // Publish block k: wait for this wave's octet, zero it if its table entry was out of
      // range, barrier (every wave's octet of block k is in LDS and every wave is done with
      // block k - 2, whose slot then receives block k + 2, loaded during block k's S^T).
      // Returns block k's halves' state.
      // FP8: the octet was converted (and zeroed where needed) before, by `convert` in the
      // prologue or during block k - 1's S^T; only the LDS writes are waited for.
      auto publish = [&](int k) -> uint32_t {
        const bool nx = k + 2 < nblk;
        Walk nw{{0, 0}, {0, 0}};
        if (nx) nw = walk(k + 2);        // scalar table reads, consumed after the barrier
        if constexpr (!FP8) {
          if (k + 1 < nblk)
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const int sl = k % kWSlots;
        const uint32_t hok = (okq >> (2 * sl)) & 3u;
        if (!FP8 && ((hok >> (wave >> 1)) & 1u) == 0) {
          // out-of-range table entry: this octet read page 0; zero its rows (V enters the
          // products; its scores are masked).  Flagged after the piece, outside the DMA waits.
          bad_page = true;
          LDS_AS uint8_t* st = lds + sl * kWBlockBytes;
#pragma unroll
          for (int cg = 0; cg < 9; ++cg)
            *(LDS_AS u32x4_t*)(st + 4096 * cg + 1024 * wave + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (nx) {
          plan_issue(k + 2, octet_base(k + 2, nw));     // issued during block k's S^T
          const int ns = (k + 2) % kWSlots;
          okq = (okq & ~(3u << (2 * ns))) | (halves_ok(nw) << (2 * ns));
        }
        return hok;
      };
      // S^T = K Q^T for block k: lane (i, h) gets row i, tokens 8jj + 4h + r as sa[4jj + r].
      // The K operands stream through a ring of kWRing registers, each read issued kWRing
      // MFMAs ahead of its use (the scheduling barriers keep the compiler from hoisting them
      // all, which would push the query operands out of registers).  Tokens the rows must not
      // see (past the piece or the causal limit, or in a dropped half) get the score that
      // scales to -inf.
      auto scores = [&](int k, uint32_t hok) -> f32x16_t {
        LDS_AS const uint8_t* st = lds + (k % kWSlots) * kWBlockBytes;
        f32x16_t sa;
        auto kload = [&](int kk) -> bf16x8_t {
          return __builtin_bit_cast(bf16x8_t, lds_ld128(st + (kb0 ^ (32 * (kk & 3))) + 4096 * (kk >> 2)));
        };
        // the rope k-steps (kk >= 32) take their query operand from LDS, two steps ahead
        auto qload = [&](int kk) -> bf16x8_t { return __builtin_bit_cast(bf16x8_t, lds_ld128(qrope + 1024 * (kk - 32))); };
        bf16x8_t kr[kWRing], qr[2];
        // FP8: block k + 1's octet is converted between the S^T steps (no vector work competes
        // there): its loads are waited for at step kWCvWait (block k + 2's are issued later),
        // then the scales and one code pair at a time
        const bool cv = FP8 && k + 1 < nblk;
        const bool cv_ok = ((okq >> (2 * ((k + 1) % kWSlots) + (wave >> 1))) & 1u) != 0;
        u32x4_t cvs, cvr;
#pragma unroll
        for (int j = 0; j < kWRing; ++j) kr[j] = kload(j);
#pragma unroll
        for (int kk = 0; kk < kKSteps * 2; ++kk) {
          if constexpr (FP8) {
            if (cv) {
              if (kk == kWCvWait) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // only block k + 1's loads are in flight
                bad_page |= !cv_ok;
                cvs = cv_scales(k + 1);
              }
              constexpr int r0 = kWCvWait + 1, w0 = r0 + kWCvLag;
              if (kk >= r0 && kk < r0 + 4 * kWCvStride && (kk - r0) % kWCvStride == 0)
                cvr = cv_read(k + 1, (kk - r0) / kWCvStride);
              if (kk >= w0 && kk < w0 + 4 * kWCvStride && (kk - w0) % kWCvStride == 0)
                cv_write(k + 1, (kk - w0) / kWCvStride, cvr, cvs, cv_ok);
            }
          }
          if (k + 2 < nblk) {                 // block k + 2's loads, one every few steps
            constexpr int d0 = FP8 ? kWDma0F8 : kWDma0, ds = FP8 ? kWDmaStrideF8 : kWDmaStride;
            constexpr int nd = FP8 ? kWF8Loads : 9;
            if (kk >= d0 && (kk - d0) % ds == 0 && (kk - d0) / ds < nd) issue_part((kk - d0) / ds);
          }
          if (kk == 30 || kk == 31) qr[kk & 1] = qload(kk + 2);
          const bf16x8_t qv = kk < 32 ? qf[kk & 31] : qr[kk & 1];
          if (kk == 0)
            mfma32_vfirst(sa, kr[0], qv);
          else if (kk == kKSteps * 2 - 1)
            mfma32_vlast(sa, kr[kk % kWRing], qv);
          else
            mfma32_vacc(sa, kr[kk % kWRing], qv);
          if (kk + kWRing < kKSteps * 2) kr[kk % kWRing] = kload(kk + kWRing);
          if (kk >= 32 && kk + 2 < kKSteps * 2) qr[kk & 1] = qload(kk + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        const int tok0 = tb + kWBlock * k;
        if (hok != 3u || tok0 + kWBlock > lim_min) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int t = tok0 + 8 * (q >> 2) + 4 * h + (q & 3);
            if (!(t < lim && ((hok >> (q >> 3)) & 1u) != 0)) sa[q] = s_hide;   // position 8 (q / 4) + ..: half q / 8
          }
        }
        return sa;
      };
      // softmax of one block's scores: p = exp2(s c - m_ref) (c = scale * log2 e), summed into
      // lsum, returned as bf16 P^T operands for the two token halves u (K index 8h + 4jp + r is
      // token 16u + 8jp + 4h + r, held in sa[8u + 4jp + r]); pl: the bf16 remainders (fp32 output)
      auto softmax = [&](const f32x16_t& sa, bool first, u32x4_t (&ph)[2], u32x4_t (&pl)[2]) {
        // sc is rounded before both the maximum and exp2(sc - m_ref) (no fused multiply-add), so
        // the row's largest score gets a weight of exactly 1
#pragma clang fp contract(off)
        float sc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) sc[q] = sa[q] * c_log2;
        float mx = sc[0];
#pragma unroll
        for (int q = 1; q < 16; ++q) mx = fmaxf(mx, sc[q]);
        {
          const int xi = __float_as_int(mx);
          const auto sw = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
          mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
        }
        m_run = fmaxf(m_run, mx);
        if (first) m_ref = fmaxf(mx, kNegBig);
        ovf |= mx > m_ref + kWSlack;
        float pv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          pv[q] = __builtin_amdgcn_exp2f(sc[q] - m_ref);
          lsum += pv[q];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float a0 = pv[8 * u + 2 * e2], a1 = pv[8 * u + 2 * e2 + 1];
            ph[u][e2] = bf16x2_rne(a0, a1);
            if constexpr (OUT_F32)
              pl[u][e2] = bf16x2_rne(a0 - __uint_as_float(ph[u][e2] << 16), a1 - __uint_as_float(ph[u][e2] & 0xFFFF0000u));
          }
        }
      };
      // O^T += V^T P^T for block kp (P^T in php / plp), with the softmax of the next block's
      // scores sa spread over its 2 NC steps (step t: token half u = t / NC, this wave's tile
      // tile0 + t % NC).  V^T tiles stream through a ring of kWVRing operands; each step is one
      // MFMA (two with fp32 output), the next tile's two transpose reads and slices of the
      // softmax (29 in all: one per step with 16 tiles, spread evenly otherwise), fenced so that
      // the compiler keeps this order (the MFMAs then run under the softmax's vector work).
      auto update = [&](int kp, const u32x4_t (&php)[2], const u32x4_t (&plp)[2], const f32x16_t& sa,
                        u32x4_t (&ph)[2], u32x4_t (&pl)[2]) {
        constexpr int T = 2 * NC;
        // tile0 is even: its column pair starts 4096 (tile0 / 2) into the block
        LDS_AS const uint8_t* st = lds + (kp % kWSlots) * kWBlockBytes + 2048 * tile0;
        auto vload = [&](int t) -> bf16x8_t {
          const int u = t / NC, cc = t % NC;
          const int off = 4096 * (cc >> 1) + 2048 * u;
          const u32x2_t v0 = lds_tr16(st + (vb[0] ^ (64 * (cc & 1))) + off);
          const u32x2_t v1 = lds_tr16(st + (vb[1] ^ (64 * (cc & 1))) + off);
          return __builtin_bit_cast(bf16x8_t, u32x4_t{v0[0], v0[1], v1[0], v1[1]});
        };
        bf16x8_t vr[kWVRing];
#pragma unroll
        for (int j = 0; j < kWVRing; ++j) vr[j] = vload(j);
        float sc[16], mx = -INFINITY;
        auto slice = [&](int sl) {
#pragma clang fp contract(off)
          if (sl < 4) {
#pragma unroll
            for (int q = 4 * sl; q < 4 * sl + 4; ++q) {
              sc[q] = sa[q] * c_log2;
              mx = fmaxf(mx, sc[q]);
            }
          } else if (sl == 4) {
            const int xi = __float_as_int(mx);
            const auto sw = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
            mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
            m_run = fmaxf(m_run, mx);
            ovf |= mx > m_ref + kWSlack;
          } else if (sl < 21) {
            const int q = sl - 5;
            sc[q] = __builtin_amdgcn_exp2f(sc[q] - m_ref);
            lsum += sc[q];
          } else if (sl < 29) {
            const int e = sl - 21, uu = e >> 2, e2 = e & 3;      // pair e2 of half uu
            const float a0 = sc[8 * uu + 2 * e2], a1 = sc[8 * uu + 2 * e2 + 1];
            ph[uu][e2] = bf16x2_rne(a0, a1);
            if constexpr (OUT_F32)
              pl[uu][e2] = bf16x2_rne(a0 - __uint_as_float(ph[uu][e2] << 16), a1 - __uint_as_float(ph[uu][e2] & 0xFFFF0000u));
          }
        };
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int u = t / NC, cc = t % NC;
          const bf16x8_t vv = vr[t % kWVRing];
          o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, __builtin_bit_cast(bf16x8_t, php[u]), o[cc], 0, 0, 0);
          if constexpr (OUT_F32)
            o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, __builtin_bit_cast(bf16x8_t, plp[u]), o[cc], 0, 0, 0);
          if (t + kWVRing < T) vr[t % kWVRing] = vload(t + kWVRing);
          // the softmax slices of this step
          const int s0 = T == 32 ? t : 29 * t / T, s1 = T == 32 ? t + 1 : 29 * (t + 1) / T;
#pragma unroll
          for (int sl = s0; sl < s1; ++sl) slice(sl);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      u32x4_t ph_prev[2], pl_prev[2];
      if constexpr (FP8) {
        if (nblk > 0) {
          // block 0's octet (block 1's loads may still be in flight)
          if (nblk > 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWF8Loads) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          const bool ok0 = ((okq >> (wave >> 1)) & 1u) != 0;
          bad_page |= !ok0;
          const u32x4_t scl = cv_scales(0);
#pragma unroll
          for (int j = 0; j < 4; ++j) cv_write(0, j, cv_read(0, j), scl, ok0);
        }
      }
      if (nblk > 0) {
        const uint32_t hok = publish(0);
        const f32x16_t sa = scores(0, hok);
        softmax(sa, pass == 0, ph_prev, pl_prev);
      }
      for (int k = 1; k <= nblk; ++k) {
        f32x16_t sa;
        if (k < nblk) {
          const uint32_t hok = publish(k);
          sa = scores(k, hok);
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) sa[q] = s_hide;       // past the last block: no weight
        }
        u32x4_t ph[2], pl[2];
        update(k - 1, ph_prev, pl_prev, sa, ph, pl);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          ph_prev[u] = ph[u];
          pl_prev[u] = pl[u];
        }
      }
      // any wave whose scores left the slack: every wave runs the piece again (the slots are
      // shared); the second pass starts from each row's true maximum and cannot overflow.  The
      // waves' votes go through slot 0, free once every wave has passed this barrier.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (lane == 0) lds[wave] = __any(ovf) ? 1 : 0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint32_t again = *(LDS_AS const uint32_t*)lds;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (again == 0 || pass > 0) break;
    }
    {
        // ---- write: every wave holds its 32 rows complete
        float l = lsum;
        {
          const int xi = __float_as_int(l);
          const auto sw = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
          l = __int_as_float(sw[0]) + __int_as_float(sw[1]);
        }
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        // lane (i, h) holds columns 32cc + 8jj + 4h + 0..3 of row i as o[cc][4jj + 0..3]; the
        // destination is the wave's first row (uniform) plus a 32-bit lane offset
        if (slot < 0 && !OUT_F32) {
          uint8_t* dst = (uint8_t*)((uint16_t*)a.out + ((int64_t)b * R + rbase) * kDv + 32 * tile0);
          const uint32_t lo = (uint32_t)i * (2 * kDv) + 8u * h;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              *(u32x2_t*)(dst + lo + 64 * cc + 16 * jj) =
                  u32x2_t{bf16x2_rne(o[cc][4 * jj] * inv, o[cc][4 * jj + 1] * inv),
                          bf16x2_rne(o[cc][4 * jj + 2] * inv, o[cc][4 * jj + 3] * inv)};
            __builtin_amdgcn_sched_barrier(0);   // one tile at a time out of the accumulators
          }
        } else {
          uint8_t* dst = (uint8_t*)((slot < 0 ? (float*)a.out + ((int64_t)b * R + rbase) * kDv
                                              : a.part_o + ((int64_t)slot * R + rbase) * kDv) + 32 * tile0);
          const uint32_t lo = (uint32_t)i * (4 * kDv) + 16u * h;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              *(f32x4_t*)(dst + lo + 128 * cc + 32 * jj) =
                  f32x4_t{o[cc][4 * jj], o[cc][4 * jj + 1], o[cc][4 * jj + 2], o[cc][4 * jj + 3]} * inv;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (h == 0 && wave % CW == 0) {     // the CW waves of a row set hold the same m and l
          const float lse = l > 0.f ? (m_ref + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
          float* lbase = slot < 0 ? a.lse + ((int64_t)b * R + rbase) : a.part_lse + ((int64_t)slot * R + rbase);
          if (slot >= 0 || a.lse) *(float*)((uint8_t*)lbase + 4u * (uint32_t)i) = lse;
        }
        if (bad_page && lane == 0)
          __hip_atomic_fetch_or(a.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


// ---------------------------------------------------------------------------------------------
// 32-row split-decode kernel (R = 32 per work-group, two-token queries over 16 heads): the token
// split of the 16-row kernel -- each wave takes blocks w, w + 4, ... of the piece through two
// LDS stages of its own -- with all 32 query rows in every wave, so one work-group reads each KV
// row once for 32 rows (two 16-row work-groups read it twice, the second time from L2).
//   S^T = K Q^T     two 16x16x32 tiles (rows 0..15, 16..31) sharing each K operand: 36 MFMAs
//   P^T             per tile exp2(s - m), moved into the 32x32x16 B-operand layout with one
//                   v_permlane16_swap per dword (lane (i, h): row i, tokens 8h .. 8h + 7)
//   O^T += V^T P^T  M = 32 columns, N = 32 rows, K = 16 tokens: 16 MFMAs (32 with fp32 output);
//                   O^T (512 x 32) fills the 256 accumulation registers
// The query's first 10 k-steps stay in VGPRs; its last 8 (192 latent and the 64 rope columns, the
// same for every wave) sit in the 16 KB of LDS beside the stages.  K and V^T operands stream
// through small register rings; a wave's stage is refilled with its block after next when the
// block's last V^T read has been issued.  Weights are taken against a per-row reference without
// rescaling (as in the 128-row kernel; a wave whose scores leave the slack runs its blocks again).
// When a piece ends the four waves' states are combined through LDS, 16 rows at a time.
// S^T steps on a 16x16x32 bf16 MFMA with the accumulator in VGPRs (O^T holds all 256
// accumulation registers): acc = a b, acc += a b, and the last step with 16 wait states so
// that vector instructions may read acc right after it.
__device__ __forceinline__ void mfma16_vfirst(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_vacc(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_vlast(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(acc) : "v"(a), "v"(b));
}

constexpr int k32QReg = 10;                              // query k-steps in VGPRs
#ifndef MLA_K32_WAVES
#define MLA_K32_WAVES 2
#endif
constexpr int k32Waves = MLA_K32_WAVES;                  // waves per work-group
constexpr int k32QLds = kSmemBytes;                      // after the 4 x 2 stages: [8 k-steps][2 tiles][64 lanes] x 16 B
constexpr int k32Smem = k32QLds + (kKSteps - k32QReg) * 2 * 1024;   // 163,840: all of the LDS

// NW waves per work-group (2 or 4) share the 8 block stages: 8 / NW each, so a wave has
// 8 / NW - 1 blocks in flight while it computes one.
template <bool OUT_F32, int NW>
__global__ void __launch_bounds__(64 * NW, 1) split32_decode_kernel(DecodeArgs a) {
  static_assert(NW == 2 || NW == 4, "2 or 4 waves");
  constexpr int SPW = 2 * kWaves / NW;             // stages per wave
  constexpr int NT = 64 * NW;                      // threads
  __shared__ __attribute__((aligned(1024))) uint8_t smem[k32Smem];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;          // S^T tile layout: row n of the tile, tokens 4g .. 4g + 3
  int worker, rgroup;
  if (a.row_groups == 1) {
    worker = blockIdx.x;
    rgroup = 0;
  } else {
    // the row groups of one token range land on the same XCD (ids are dealt round-robin to 8 XCDs)
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    rgroup = y % a.row_groups;
    worker = (y / a.row_groups) * 8 + x;
  }
  if (worker >= a.num_workers) return;
  const int R = a.rows;
  const int row0 = 32 * rgroup;                    // this work-group's 32 query rows
  const bool stream = a.row_groups == 1;           // KV loads: non-temporal when no other row group re-reads

  // Block layout (as the 16-row kernel): chunk c of token t at 2048 (c / 8) + 128 t + 16 ((c % 8) ^ row_swz(t)).
  // K, k-step kk: token n, chunk 4 kk + g.
  const int k_even = 128 * n + 16 * (g ^ row_swz(n));
  const int k_odd = k_even ^ 64;
  // V^T, 32-column tile cc, part jp: lane 4e + qq of 16-lane group g reads token 8 (g / 2) + 4 jp + e,
  // columns 32 cc + 16 (g % 2) + 4 qq .. + 3 (chunk 4 cc + 2 (g % 2) + qq / 2, 8 B); the transpose
  // hands lane (i, h) column 32 cc + i of tokens 8 h + 4 jp + 0 .. 3.
  int v_off[2][2];       // [cc % 2][jp]; + 2048 (cc / 2)
  {
    const int e = n >> 2, qq = n & 3;
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const int t = 8 * (g >> 1) + 4 * jp + e;
        const int c = 4 * par + 2 * (g & 1) + (qq >> 1);
        v_off[par][jp] = 128 * t + 16 * (c ^ row_swz(t)) + 8 * (qq & 1);
      }
  }
  const int ld_tok0 = lane >> 3, ld_tok1 = 8 + (lane >> 3);
  const int ld_col0 = 8 * ((lane & 7) ^ row_swz(ld_tok0)), ld_col1 = 8 * ((lane & 7) ^ row_swz(ld_tok1));
  LDS_AS uint8_t* const stages = lds + wave * SPW * kBlockBytes;   // this wave's SPW stages
  LDS_AS uint8_t* const qlds = lds + k32QLds + 16 * lane;      // + 1024 (2 (kk - k32QReg) + tile)

  const CST_AS int32_t* worker_off = as_const(a.worker_off);
  const CST_AS int32_t* pieces = as_const(a.pieces);
  const CST_AS int32_t* seqlens = as_const(a.seqlens);
  const CST_AS int32_t* block_table = as_const(a.block_table);

  // the piece range is read with the plan id, the pieces once the id matches
  const int p_begin = worker_off[worker], p_end = worker_off[worker + 1];
  if (!schedule_matches(a)) return;
  for (int pi = p_begin; pi < p_end; ++pi) {
    const int b = pieces[4 * pi + 0], tb = pieces[4 * pi + 1], slot = pieces[4 * pi + 3];
    check_planned_length(a, b, pieces[4 * pi + 2], seqlens[b]);
    const int L = seqlens[b];
    const int te = min(pieces[4 * pi + 2], L);
    const int nblk = te > tb ? (te - tb + kBlock - 1) / kBlock : 0;
    // the tokens row 16 t + n sees (causal: the first L - (q_len - 1 - row / num_heads))
    int lim[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) lim[t] = a.causal ? min(te, L - (a.q_len - 1 - (row0 + 16 * t + n) / a.num_heads)) : te;
    const int my_n = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
    auto blk_of = [&](int k) { return wave + NW * k; };

    // query rows as B operands: lane (n, g) holds row 16 t + n, columns 32 kk + 8 g .. + 7; k-steps
    // below k32QReg in VGPRs, the others in LDS (wave w writes k-steps k32QReg + (8 / NW) w ..;
    // every wave reads all of them after the barrier below)
    bf16x8_t qf[2][k32QReg];
    {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* qrow = a.q + ((int64_t)b * R + row0 + 16 * t + n) * kDqk + 8 * g;
#pragma unroll
        for (int kk = 0; kk < k32QReg; ++kk) qf[t][kk] = *(const bf16x8_t*)(qrow + 32 * kk);
#pragma unroll
        for (int j = 0; j < (kKSteps - k32QReg) / NW; ++j) {
          const int kk = k32QReg + (kKSteps - k32QReg) / NW * wave + j;
          *(LDS_AS u32x4_t*)(qlds + 1024 * (2 * (kk - k32QReg) + t)) = *(const u32x4_t*)(qrow + 32 * kk);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): the query loads (a wait the compiler sees)
    }
    __syncthreads();

    float m_ref[2], lsum[2];                 // reference max per tile row (log2 units); this lane's share of sum p
    float m_run[2] = {-INFINITY, -INFINITY}; // the row's largest scaled score so far
    bool bad_page = false;                   // a block of this wave read an out-of-range table entry
    f32x16_t o[16];

    struct Src {
      const uint8_t* row0;
      uint32_t vo[2];
    };
    auto source = [&](int k, bool& ok) -> Src {
      const int tok0 = tb + kBlock * blk_of(k);
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.page_shift, a.num_pages, b, tok0);
      ok = base >= 0;
      if (!ok) base = 0;
      const int last = te - 1 - tok0;
      Src r{};
      r.row0 = (const uint8_t*)(a.kv + base * kDqk);
      r.vo[0] = (uint32_t)(min(ld_tok0, last) * kRowBytesBf16 + 2 * ld_col0);
      r.vo[1] = (uint32_t)(min(ld_tok1, last) * kRowBytesBf16 + 2 * ld_col1);
      return r;
    };
    auto issue = [&](const Src& src, LDS_AS uint8_t* stage) {
      const uint32_t l = (uint32_t)(uintptr_t)stage;
      if (stream)
        dma_bf16_block<true>(src.row0, src.vo[0], src.vo[1], l);
      else
        dma_bf16_block<false>(src.row0, src.vo[0], src.vo[1], l);
    };
    // P^T for the 32x32x16 MFMA from the tiles' weights (lane (n, g): row 16 t + n, tokens
    // 4g .. 4g + 3, packed as two bf16x2 words): one permlane16_swap per word gives lane (i, h)
    // the words of row i, tokens 8h .. 8h + 3 (first) and 8h + 4 .. 8h + 7 (second).
    auto pt_operand = [&](const uint32_t (&w0)[2], const uint32_t (&w1)[2]) -> bf16x8_t {
      const auto s0 = __builtin_amdgcn_permlane16_swap(w0[0], w1[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(w0[1], w1[1], false, false);
      return __builtin_bit_cast(bf16x8_t, u32x4_t{s0[0], s1[0], s0[1], s1[1]});
    };
    // O^T += V^T P^T with p = exp2(s - m_ref); fp32 output: p as bf16 hi + lo, two MFMAs per tile.
    // The V^T operands of stage st stream through a ring of three, each read three MFMAs ahead.
    auto vload = [&](LDS_AS const uint8_t* st, int cc) -> bf16x8_t {
      const u32x2_t v0 = lds_tr16(st + 2048 * (cc >> 1) + v_off[cc & 1][0]);
      const u32x2_t v1 = lds_tr16(st + 2048 * (cc >> 1) + v_off[cc & 1][1]);
      return __builtin_bit_cast(bf16x8_t, u32x4_t{v0[0], v0[1], v1[0], v1[1]});
    };
    auto accumulate = [&](const float (&s)[2][4], LDS_AS const uint8_t* st) {
      uint32_t hw[2][2], lw[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          p[q] = __builtin_amdgcn_exp2f(s[t][q] - m_ref[t]);
          lsum[t] += p[q];
        }
        const u32x4_t hl = split_hi_lo(p[0], p[1], p[2], p[3]);
        hw[t][0] = hl[0];
        hw[t][1] = hl[1];
        lw[t][0] = hl[2];
        lw[t][1] = hl[3];
      }
      const bf16x8_t ph = pt_operand(hw[0], hw[1]);
      bf16x8_t pl;
      if constexpr (OUT_F32) pl = pt_operand(lw[0], lw[1]);
      constexpr int kVRing = 3;
      bf16x8_t vr[kVRing];
#pragma unroll
      for (int j = 0; j < kVRing; ++j) vr[j] = vload(st, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const bf16x8_t vv = vr[cc % kVRing];
        if (cc + kVRing < 16) vr[cc % kVRing] = vload(st, cc + kVRing);
        o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, ph, o[cc], 0, 0, 0);
        if constexpr (OUT_F32) o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pl, o[cc], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Weights without rescaling (as the 128-row kernel): each row's reference is the maximum of
    // this wave's first block; a wave whose later scores exceed it by more than kWSlack runs its
    // blocks again with the true maximum, so the accumulators are only ever touched by MFMAs.
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[c][q] = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        m_ref[t] = pass ? fmaxf(m_run[t], kNegBig) : kNegBig;
        lsum[t] = 0.f;
      }
      bool have_ref = pass > 0, ovf = false;
      uint32_t okq = 0;              // bit s: the table entry of the block now in stage s was in range
#pragma unroll
      for (int s0 = 0; s0 < SPW; ++s0) {
        bool ok = true;
        if (s0 < my_n) issue(source(s0, ok), stages + s0 * kBlockBytes);
        okq |= (ok ? 1u : 0u) << s0;
      }
      for (int k = 0; k < my_n; ++k) {
        const int sl = k % SPW;
        LDS_AS uint8_t* st = stages + sl * kBlockBytes;
        bool nok = true;
        const bool nx = k + SPW < my_n;
        Src nsrc{};
        if (nx) nsrc = source(k + SPW, nok);
        // block k has landed once at most the loads of the blocks after it are in flight
        const int after = min(SPW - 1, my_n - 1 - k);
        if (after >= 3)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kLoadsPerBlock) : "memory");
        else if (after == 2)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLoadsPerBlock) : "memory");
        else if (after == 1)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerBlock) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const bool ok = (okq >> sl) & 1u;
        okq = (okq & ~(1u << sl)) | ((nok ? 1u : 0u) << sl);   // the stage's next occupant
        if (!ok) {
          // out-of-range table entry: the block read page 0; it takes the same path with its rows
          // zeroed (V enters the products) and every score masked, so the accumulators keep one
          // definition per step
          bad_page = true;
#pragma unroll
          for (int u = 0; u < kBlockBytes / 1024; ++u)
            *(LDS_AS u32x4_t*)(st + 1024 * u + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
        }
        // S^T with the K operands streamed
        f32x4_t sacc[2];
        {
          auto kload = [&](int kk) -> bf16x8_t {
            return __builtin_bit_cast(bf16x8_t, lds_ld128(st + ((kk & 1) ? k_odd : k_even) + 2048 * (kk >> 1)));
          };
          // the query operands in LDS are the same for every block: an address the compiler cannot
          // see through keeps it from hoisting their loads out of the block loop (into registers)
          uint32_t qa = (uint32_t)(uintptr_t)qlds;
          asm volatile("" : "+v"(qa));
          LDS_AS const uint8_t* const qb = (LDS_AS const uint8_t*)(uintptr_t)qa;
          auto qload = [&](int kk, int t) -> bf16x8_t {
            return __builtin_bit_cast(bf16x8_t, lds_ld128(qb + 1024 * (2 * (kk - k32QReg) + t)));
          };
          constexpr int kRing = 4;
          bf16x8_t kr[kRing], qr[2][2];        // K: kRing steps ahead; LDS query operands: two steps ahead
#pragma unroll
          for (int j = 0; j < kRing; ++j) kr[j] = kload(j);
#pragma unroll
          for (int kk = 0; kk < kKSteps; ++kk) {
            const bf16x8_t kv = kr[kk % kRing];
            if (kk + kRing < kKSteps) kr[kk % kRing] = kload(kk + kRing);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const bf16x8_t qv = kk < k32QReg ? qf[t][kk < k32QReg ? kk : 0] : qr[kk & 1][t];
              if (kk == 0)
                mfma16_vfirst(sacc[t], kv, qv);
              else if (kk == kKSteps - 1)
                mfma16_vlast(sacc[t], kv, qv);
              else
                mfma16_vacc(sacc[t], kv, qv);
            }
            if (kk + 2 >= k32QReg && kk + 2 < kKSteps) {     // (after this step's use of the slot)
#pragma unroll
              for (int t = 0; t < 2; ++t) qr[kk & 1][t] = qload(kk + 2, t);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        const int tok0 = tb + kBlock * blk_of(k);
        float sc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int nvalid = ok ? lim[t] - tok0 : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) sc[t][q] = (4 * g + q < nvalid) ? sacc[t][q] * a.scale_log2 : -INFINITY;
          const float mx = wave_max_over_groups(fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3])));
          m_run[t] = fmaxf(m_run[t], mx);
          if (!have_ref) m_ref[t] = fmaxf(mx, kNegBig);
          ovf |= mx > m_ref[t] + kWSlack;
        }
        have_ref = true;
        accumulate(sc, st);
        if (nx) issue(nsrc, st);        // every read of the stage has been issued (the load waits for them)
      }
      if (pass > 0 || !__any(ovf)) break;
    }

    if (bad_page && lane == 0)
      __hip_atomic_fetch_or(a.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // ---- combine the waves' states and write.  NW / 2 rounds through LDS: waves 2 r, 2 r + 1
    // write all 32 rows (so that every wave reads its accumulators once), then thread (row
    // tid / SEG, columns 4 (tid % SEG) + 4 SEG j) folds them into its running sum.
    const int i = lane & 31;
    float m_o, l_o;                        // this lane's O^T row i: its reference and weight sum
    {
      const float l0 = wave_sum_over_groups(lsum[0]), l1 = wave_sum_over_groups(lsum[1]);
      const float ma = __shfl(m_ref[0], i & 15), mb = __shfl(m_ref[1], i & 15);
      const float la = __shfl(l0, i & 15), lb = __shfl(l1, i & 15);
      m_o = i < 16 ? ma : mb;
      l_o = i < 16 ? la : lb;
    }
    __syncthreads();   // stages no longer read
    LDS_AS float* buf = (LDS_AS float*)smem;                     // [2 waves][32 rows][516]
    LDS_AS float* sm_m = buf + 2 * 32 * kMergeStride;            // [2][32]
    LDS_AS float* sm_l = sm_m + 64;                              // [2][32]
    constexpr int SEG = NT / 32;                 // threads per row
    constexpr int NCOL = kDv / (4 * SEG);        // float4 columns per thread
    const int r = threadIdx.x / SEG, seg = threadIdx.x % SEG;
    f32x4_t acc[NCOL];
    float M = kNegBig, Ls = 0.f;
#pragma unroll
    for (int round = 0; round < NW / 2; ++round) {
      if ((wave >> 1) == round) {
        const int w2 = wave & 1;
        if (lane < 32) {
          sm_m[32 * w2 + i] = m_o;
          sm_l[32 * w2 + i] = l_o;
        }
        // lane (i, h): row i, columns 32 cc + 8 jj + 4 h + 0..3 in o[cc][4 jj + 0..3]
        LDS_AS float* my = buf + (32 * w2 + i) * kMergeStride + 4 * (lane >> 5);
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *(LDS_AS f32x4_t*)(my + 32 * cc + 8 * jj) = f32x4_t{o[cc][4 * jj], o[cc][4 * jj + 1], o[cc][4 * jj + 2], o[cc][4 * jj + 3]};
          __builtin_amdgcn_sched_barrier(0);   // one tile at a time out of the accumulators
        }
      }
      __syncthreads();
      const float m0 = sm_m[r], m1 = sm_m[32 + r];
      const float Mn = fmaxf(M, fmaxf(m0, m1));
      const float fa = M <= kNegBig ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float f0 = m0 <= kNegBig ? 0.f : __builtin_amdgcn_exp2f(m0 - Mn);
      const float f1 = m1 <= kNegBig ? 0.f : __builtin_amdgcn_exp2f(m1 - Mn);
      Ls = Ls * fa + f0 * sm_l[r] + f1 * sm_l[32 + r];
#pragma unroll
      for (int j = 0; j < NCOL; ++j) {
        const int d = 4 * seg + 4 * SEG * j;
        const f32x4_t x0 = *(LDS_AS const f32x4_t*)(buf + r * kMergeStride + d);
        const f32x4_t x1 = *(LDS_AS const f32x4_t*)(buf + (32 + r) * kMergeStride + d);
        acc[j] = round == 0 ? f0 * x0 + f1 * x1 : acc[j] * fa + f0 * x0 + f1 * x1;
      }
      M = Mn;
      __syncthreads();
    }
    const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
#pragma unroll
    for (int j = 0; j < NCOL; ++j) {
      const int d = 4 * seg + 4 * SEG * j;
      const f32x4_t v = acc[j] * inv;
      if (slot < 0) {
        const int64_t off = ((int64_t)b * R + row0 + r) * kDv + d;
        if (OUT_F32) {
          *(f32x4_t*)((float*)a.out + off) = v;
        } else {
          *(u32x2_t*)((uint16_t*)a.out + off) = u32x2_t{bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
        }
      } else {
        *(f32x4_t*)(a.part_o + ((int64_t)slot * R + row0 + r) * kDv + d) = v;
      }
    }
    if (seg == 0) {
      const float lse = Ls > 0.f ? (M + __log2f(Ls)) * 0.69314718055994530942f : -INFINITY;
      if (slot < 0) {
        if (a.lse) a.lse[(int64_t)b * R + row0 + r] = lse;
      } else {
        a.part_lse[(int64_t)slot * R + row0 + r] = lse;
      }
    }
  }
}

// Merge of split sequences.  One work-group per (sequence, 16 query rows, 64
// output columns): thread (r, q) merges row r, columns 4q..4q+3 of the slice over
// all of the sequence's partial results, so every partial byte is read once and
// all loads of a thread are independent.
constexpr int kMergeCols = 64;
template <bool OUT_F32, int NB>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  // The plan id in the workspace is read alongside the first loads rather than before them:
  // the workspace is at least this plan's size (the host checks it), so the merge table and,
  // with the uniform layout, the partials are in bounds whatever schedule it holds.  Table
  // entries are used as addresses, and anything is stored, only once the id matches (another
  // plan's schedule: the split launch flagged it).
  const uint64_t pid = *as_const(a.ws_plan_id);
  const int R = a.rows;
  const int col_groups = kDv / kMergeCols;
  const int per_item = (R / 16) * col_groups;
  const int item = blockIdx.x / per_item;
  const int rem = blockIdx.x % per_item;
  const int rg = rem / col_groups, cg = rem % col_groups;
  int b, s0, ns;
  if (a.uniform_ns > 0) {          // item i is sequence i with slots [i*ns, (i+1)*ns): no table read
    b = item;
    s0 = item * a.uniform_ns;
    ns = a.uniform_ns;
  } else {
    const CST_AS int32_t* merges = as_const(a.merges);
    b = merges[4 * item + 0];
    s0 = merges[4 * item + 1];
    ns = merges[4 * item + 2];
    asm volatile("" ::"s"(b), "s"(s0), "s"(ns));    // the table reads go out with the id's
    if (pid != a.plan_id) return;
  }
  const int r = rg * 16 + (threadIdx.x >> 4);
  const int d = cg * kMergeCols + 4 * (threadIdx.x & 15);
  const float* lse_col = a.part_lse + (int64_t)s0 * R + r;                 // stride R per slot
  const float* o_col = a.part_o + ((int64_t)s0 * R + r) * kDv + d;         // stride R*512 per slot
  // one pass: NB partial results (their lse and 4 columns of o) are loaded at once, so the
  // loads of a batch overlap; the running max moves per batch.  NB is the plan's largest piece
  // count rounded up to 4, 8 or 16: a smaller batch holds fewer registers, so more waves (and
  // more loads) are resident when there are many sequences with few pieces each.
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; s += NB) {
    float l[NB];
    f32x4_t v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool in = s + u < ns;
      l[u] = in ? lse_col[(int64_t)(s + u) * R] : -INFINITY;
      v[u] = in ? *(const f32x4_t*)(o_col + (int64_t)(s + u) * R * kDv) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    merge_batch<NB>(l, v, M, L, acc);
  }
  if (pid != a.plan_id) return;
  const f32x4_t v = acc * (L > 0.f ? 1.0f / L : 0.f);
  const int64_t off = ((int64_t)b * R + r) * kDv + d;
  if (OUT_F32) {
    *(f32x4_t*)((float*)a.out + off) = v;
  } else {
    u32x2_t pkd;
    pkd[0] = bf16x2_rne(v[0], v[1]);
    pkd[1] = bf16x2_rne(v[2], v[3]);
    *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
  }
  if (cg == 0 && (threadIdx.x & 15) == 0 && a.lse) a.lse[(int64_t)b * R + r] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// Merge for the device schedule: one work-group per (sequence, 16 rows, 64 columns), as
// merge_kernel, with the sequence's pieces taken from the cut its first piece recorded
// (seq_info[b] = {first work-group or -1 if not split, last work-group, 1 if the first
// piece starts inside its work-group's range}; seq_info[4B..4B+1] = T, W).
template <bool OUT_F32>
__global__ void __launch_bounds__(256) merge_dev_kernel(MergeArgs a) {
  const int R = a.rows;
  const int col_groups = kDv / kMergeCols;
  const int per_seq = (R / 16) * col_groups;
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x % per_seq;
  const int rg = rem / col_groups, cg = rem % col_groups;
  const CST_AS int32_t* info = as_const(a.seq_info);
  const int wf = info[4 * b + 0], wl = info[4 * b + 1], first_inside = info[4 * b + 2];
  if (wf < 0) return;
  const int64_t T = info[4 * a.batch + 0];
  const int W = info[4 * a.batch + 1];
  auto wstart = [&](int w) { return T * w / W; };
  auto slot_of = [&](int w) -> int {
    return wstart(w + 1) > wstart(w) ? 2 * w + (w == wf ? first_inside : 0) : -1;
  };
  const int r = rg * 16 + (threadIdx.x >> 4);
  const int d = cg * kMergeCols + 4 * (threadIdx.x & 15);
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int w0 = wf; w0 <= wl; w0 += kMergeBatch) {
    float l[kMergeBatch];
    f32x4_t v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int sl = w0 + u <= wl ? slot_of(w0 + u) : -1;
      l[u] = sl >= 0 ? a.part_lse[(int64_t)sl * R + r] : -INFINITY;
      v[u] = sl >= 0 ? *(const f32x4_t*)(a.part_o + ((int64_t)sl * R + r) * kDv + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    merge_batch(l, v, M, L, acc);
  }
  const f32x4_t v = acc * (L > 0.f ? 1.0f / L : 0.f);
  const int64_t off = ((int64_t)b * R + r) * kDv + d;
  if (OUT_F32) {
    *(f32x4_t*)((float*)a.out + off) = v;
  } else {
    u32x2_t pkd;
    pkd[0] = bf16x2_rne(v[0], v[1]);
    pkd[1] = bf16x2_rne(v[2], v[3]);
    *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
  }
  if (cg == 0 && (threadIdx.x & 15) == 0 && a.lse) a.lse[(int64_t)b * R + r] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// Debug gather: one thread per 16-B chunk of a sequence's logical rows (row_bytes per row).
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* kv, const int32_t* block_table, uint8_t* rows_out,
                                                     int32_t seq, int32_t length, int64_t row_offset,
                                                     int32_t page_size, int32_t bt_stride, int32_t num_pages,
                                                     int32_t row_bytes) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int chunks = row_bytes / 16;
  const int t = (int)(idx / chunks);
  const int c = (int)(idx % chunks);
  if (t >= length) return;
  const int64_t row = kv_row_of(block_table, bt_stride, page_size, -1, num_pages, seq, t);
  if (row < 0) return;
  *(u32x4_t*)(rows_out + (row_offset + t) * row_bytes + 16 * c) = *(const u32x4_t*)(kv + row * row_bytes + 16 * c);
}


template <bool DEV, bool COMB>
void launch_split_t(const DecodeArgs& a, bool out_fp32, int grid, hipStream_t s) {
  if (a.kv_fp8) {
    if (out_fp32)
      hipLaunchKernelGGL((split_decode_kernel<true, true, DEV, COMB>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((split_decode_kernel<false, true, DEV, COMB>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    if (out_fp32)
      hipLaunchKernelGGL((split_decode_kernel<true, false, DEV, COMB>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((split_decode_kernel<false, false, DEV, COMB>), dim3(grid), dim3(kThreads), 0, s, a);
  }
}
// a.merge_cnt set: the launch combines split sequences itself (no merge launch follows)
template <bool DEV>
void launch_split(const DecodeArgs& a, bool out_fp32, int grid, hipStream_t s) {
  if (a.merge_cnt)
    launch_split_t<DEV, true>(a, out_fp32, grid, s);
  else
    launch_split_t<DEV, false>(a, out_fp32, grid, s);
}

// The wide kernel: non-temporal KV loads when one row group reads each token range and the rows
// are bf16.  FP8 rows (656 B) are not 64-B aligned and each wave gathers its octet by region, so
// neighbouring loads share cache lines; with non-temporal loads those lines left the L2 between
// the two loads and were fetched twice (6% more HBM bytes on the ragged 128-head workload).
template <bool FP8, int CW>
void launch_wide_t(const DecodeArgs& a, bool out_fp32, int grid, hipStream_t s) {
  const bool nt = a.row_groups == 1 && !FP8;
  if (out_fp32) {
    if (nt)
      hipLaunchKernelGGL((wide_decode_kernel<true, true, FP8, CW>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((wide_decode_kernel<true, false, FP8, CW>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    if (nt)
      hipLaunchKernelGGL((wide_decode_kernel<false, true, FP8, CW>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((wide_decode_kernel<false, false, FP8, CW>), dim3(grid), dim3(kThreads), 0, s, a);
  }
}
// 128 or 64 rows per work-group: each set of 32 rows computed by one or two waves
void launch_wide(const DecodeArgs& a, int rows_per_group, bool out_fp32, int grid, hipStream_t s) {
  if (rows_per_group == 128) {
    if (a.kv_fp8) launch_wide_t<true, 1>(a, out_fp32, grid, s); else launch_wide_t<false, 1>(a, out_fp32, grid, s);
  } else {
    if (a.kv_fp8) launch_wide_t<true, 2>(a, out_fp32, grid, s); else launch_wide_t<false, 2>(a, out_fp32, grid, s);
  }
}

// Read ceiling of the decode's KV stream: every work-group moves its contiguous share of `buf`
// into LDS with the same non-temporal 16-B global->LDS loads as the decode (each wave 18 KB blocks
// through two stages, blocks w, w + 4, ... of its work-group's share) and computes nothing.
constexpr int kProbeBlock = kBlockBytes;                 // 18,432 bytes, 18 loads of 1 KB
__global__ void __launch_bounds__(kThreads) stream_probe_kernel(const uint8_t* buf, int64_t per_wg) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWaves * 2 * kProbeBlock];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* base = buf + (int64_t)blockIdx.x * per_wg;
  const int64_t nblk = per_wg / kProbeBlock;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem + (uint32_t)(wave * 2 * kProbeBlock);
  const uint32_t voff = 16u * (uint32_t)lane;
  int64_t k = 0;
  for (int64_t j = wave; j < nblk; j += kWaves, ++k) {
    const uint8_t* src = base + j * kProbeBlock;
    const uint32_t stage = lds0 + (uint32_t)((k & 1) * kProbeBlock);
#pragma unroll
    for (int i = 0; i < kProbeBlock / 1024; ++i) {
      uint32_t sv;
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\ts_mov_b32 m0, %0"
                   : "=&s"(sv)
                   : "s"(__builtin_amdgcn_readfirstlane(stage + 1024u * i)), "v"(voff), "s"(src + 1024 * i)
                   : "memory");
    }
    // the previous block has landed (18 loads per block; at most one block in flight behind)
    asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

int launch_fill_zero(void* p, size_t bytes, void* stream) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)p, n);
  return (int)hipGetLastError();
}

int launch_decode(const DecodeArgs& a, int rows_per_group, bool out_fp32, int grid, void* stream,
                  bool device_schedule) {
  hipStream_t s = (hipStream_t)stream;
  if ((rows_per_group == 128 || rows_per_group == 64) && !device_schedule) {
    launch_wide(a, rows_per_group, out_fp32, grid, s);
  } else if (device_schedule || a.kv_fp8) {
    if (rows_per_group != 16) return (int)hipErrorInvalidValue;
    if (device_schedule)
      launch_split<true>(a, out_fp32, grid, s);
    else
      launch_split<false>(a, out_fp32, grid, s);
  } else if (rows_per_group == 16) {
    launch_split<false>(a, out_fp32, grid, s);
  } else if (rows_per_group == 32) {
    if (out_fp32)
      hipLaunchKernelGGL((split32_decode_kernel<true, k32Waves>), dim3(grid), dim3(64 * k32Waves), 0, s, a);
    else
      hipLaunchKernelGGL((split32_decode_kernel<false, k32Waves>), dim3(grid), dim3(64 * k32Waves), 0, s, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_stream_probe(const void* buf, int64_t per_wg, int grid, void* stream) {
  hipLaunchKernelGGL(stream_probe_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, (const uint8_t*)buf,
                     per_wg);
  return (int)hipGetLastError();
}

int launch_merge_dev(const MergeArgs& a, bool out_fp32, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int grid = a.batch * (a.rows / 16) * (kDv / kMergeCols);
  if (grid == 0) return 0;
  if (out_fp32)
    hipLaunchKernelGGL((merge_dev_kernel<true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((merge_dev_kernel<false>), dim3(grid), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

template <int NB>
void launch_merge_t(const MergeArgs& a, bool out_fp32, int grid, hipStream_t s) {
  if (out_fp32)
    hipLaunchKernelGGL((merge_kernel<true, NB>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<false, NB>), dim3(grid), dim3(256), 0, s, a);
}
int launch_merge(const MergeArgs& a, bool out_fp32, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int grid = a.num_merges * (a.rows / 16) * (kDv / kMergeCols);
  if (a.max_ns <= 4)
    launch_merge_t<4>(a, out_fp32, grid, s);
  else if (a.max_ns <= 8)
    launch_merge_t<8>(a, out_fp32, grid, s);
  else
    launch_merge_t<16>(a, out_fp32, grid, s);
  return (int)hipGetLastError();
}

int launch_gather(const void* kv, const int32_t* block_table, void* rows_out, int32_t seq, int32_t length,
                  int64_t row_offset, int32_t page_size, int32_t bt_stride, int32_t num_pages, int32_t row_bytes,
                  void* stream) {
  const int64_t chunks = (int64_t)length * (row_bytes / 16);
  const int grid = (int)((chunks + 255) / 256);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)kv, block_table,
                     (uint8_t*)rows_out, seq, length, row_offset, page_size, bt_stride, num_pages, row_bytes);
  return (int)hipGetLastError();
}

const char* hip_error_string(int code) { return hipGetErrorString((hipError_t)code); }

// Workspace of mla_decode_devplan_noalloc: one array per GPU, held until the process ends.  In
// host code `scratch` only names the symbol; its device address comes from hipGetSymbolAddress,
// once per device with that device current, and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

int noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return 0;
}

}  // namespace mla
