// gfx950 kernels for paged MLA decode: split decode, merge of split results,
// and a debug gather that shares the decode kernel's page walk.
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

// Chunk-major block layout of the grouped kernel (16-B units): chunk c of token t sits at
// 16 * c + (t ^ ((c & 1) * kSwz)).
constexpr int kSwz = 8;

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

// Split-decode kernel: 16 query rows per work-group (R = 16 * row groups).  FP8: the cache
// rows are 656-byte fp8 rows (see kF8Row); each wave streams its blocks through three fp8
// stages and builds the MFMA operands from the codes in registers (see the FP8 loop).
// DEV: no host schedule; the work-groups cut the batch's blocks among themselves from the
// device cache_seqlens and combine split sequences in the same launch (see below).
template <bool OUT_F32, bool FP8, bool DEV>
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
          if (!ok && lane == 0) __hip_atomic_fetch_or(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            const float sc = __uint_as_float(ksc[kk >> 2]);
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
            if (lane == 0) __hip_atomic_fetch_or(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        } else {
          *(f32x4_t*)(a.part_o + ((int64_t)slot * R + grow) * kDv + d) = acc;
        }
      }
      if (dseg == 0) {
        const float lse = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
        if (slot < 0) {
          if (a.lse) a.lse[(int64_t)b * R + grow] = lse;
        } else {
          a.part_lse[(int64_t)slot * R + grow] = lse;
        }
      }
    }
    __syncthreads();
  };

  if constexpr (!DEV) {
    const int p_begin = worker_off[worker], p_end = worker_off[worker + 1];
    for (int pi = p_begin; pi < p_end; ++pi)
      run_piece(pieces[4 * pi + 0], pieces[4 * pi + 1], pieces[4 * pi + 2], pieces[4 * pi + 3]);
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

// Nine loads of one wave's share of a grouped-kernel step: load i reads 16 B per lane at
// src + 64 i and writes 1 KB at lds + 1024 i.  The instruction offset (64 i) applies to
// both addresses, so M0 steps by 960 between loads.  As dma_bf16_block: opens with
// s_waitcnt lgkmcnt(0), saves and restores M0, is hidden from the compiler's counters.
template <bool NT>
__device__ __forceinline__ void dma_group_share(const uint16_t* src, uint32_t lds) {
  uint32_t sv;
#define MLA_GROUP_DMA(NTS)                                                                        \
  asm volatile(                                                                                   \
      "s_waitcnt lgkmcnt(0)\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"               \
      "global_load_lds_dwordx4 %1, off" NTS "\n\t"                                                \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:64" NTS "\n\t"  \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:128" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:192" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:256" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:320" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:384" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:448" NTS "\n\t" \
      "s_add_u32 m0, m0, 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:512" NTS "\n\t" \
      "s_mov_b32 m0, %0"                                                                          \
      : "=&s"(sv)                                                                                 \
      : "v"(src), "s"(lds)                                                                        \
      : "memory", "scc")
  if constexpr (NT)
    MLA_GROUP_DMA(" nt");
  else
    MLA_GROUP_DMA("");
#undef MLA_GROUP_DMA
}

// Grouped split-decode kernel for 16 * RG query rows per work-group.  The four
// waves consume the same KV stream.  Each step is 32 tokens (two 16-token blocks);
// the work-group keeps four step slots in LDS (three steps in flight), filled by
// global->LDS DMA split evenly over the waves (9 loads each per step), and moves from
// step to step behind one barrier that publishes the step's data and frees the slot
// read in the previous step.
//
// RG = 4 (64 rows): wave rg owns query rows 16*rg..16*rg+15 and all 512 output columns,
// computes S^T over both blocks of the step and O^T += V^T P^T on 16x16x32 MFMA with
// K = 32 tokens.  RG = 2 (32 rows) takes the token split below.
//
// TS (token split, RG = 2 only): wave w owns rows 16 (w & 1) .. + 15, all 512 columns, and
// block w >> 1 of every step, with its own online-softmax state, so the two row groups share
// each step's LDS data without repeating S^T; the two waves of a row group are merged
// through LDS at the end of a piece.
template <int RG, bool OUT_F32, bool TS>
__global__ void __launch_bounds__(kThreads, 1) group_decode_kernel(DecodeArgs a) {
  static_assert(TS ? RG == 2 : RG == kWaves, "32 rows: token split; 64 rows: one row group per wave");
  constexpr int SB = 2;                                 // blocks per step
  constexpr int SLOTS = kWaves * kStages / SB;          // step slots (4)
  constexpr int LOADS = kLoadsPerBlock * SB / kWaves;   // DMA instructions per wave and step (9)
  constexpr int MBW = kVBlocks;                         // 16-column output blocks per wave
  static_assert(LOADS * kWaves == kLoadsPerBlock * SB && LOADS == 9 && SB == 2 && MBW % 8 == 0, "layout");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int rg = TS ? (wave & 1) : wave;
  const int th = TS ? (wave >> 1) : 0;                  // TS: the block of each step this wave takes

  int worker, rgroup;
  if (a.row_groups == 1) {
    worker = blockIdx.x;
    rgroup = 0;
  } else {
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    rgroup = y % a.row_groups;
    worker = (y / a.row_groups) * 8 + x;
  }
  if (worker >= a.num_workers) return;
  const int R = a.rows;
  const bool stream = a.row_groups == 1;   // KV loads: non-temporal when no other row group re-reads
  const int row0 = rgroup * 16 * RG + 16 * rg;

  const int k_lane = (g * 16 + (n ^ ((g & 1) * kSwz))) * 16;
  const int e = n >> 2, qq = n & 3;
  const int v_lane = ((qq >> 1) * 16 + ((4 * g + e) ^ ((qq >> 1) * kSwz))) * 16 + (qq & 1) * 8;
  const int ld_token = n ^ ((g & 1) * kSwz);

  const CST_AS int32_t* worker_off = as_const(a.worker_off);
  const CST_AS int32_t* pieces = as_const(a.pieces);
  const CST_AS int32_t* seqlens = as_const(a.seqlens);
  const CST_AS int32_t* block_table = as_const(a.block_table);

  const int p_begin = worker_off[worker], p_end = worker_off[worker + 1];
  for (int pi = p_begin; pi < p_end; ++pi) {
    const int b = pieces[4 * pi + 0];
    const int tb = pieces[4 * pi + 1];
    const int te = min(pieces[4 * pi + 2], seqlens[b]);
    const int slot = pieces[4 * pi + 3];
    const int nblk = te > tb ? (te - tb + kBlock - 1) / kBlock : 0;
    const int steps = (nblk + SB - 1) / SB;
    // end of the tokens this lane's query row sees (causal: the first L - (q_len - 1 - i))
    const int lim = a.causal ? min(te, seqlens[b] - (a.q_len - 1 - (row0 + n) / a.num_heads)) : te;

    bf16x8_t qf[kKSteps];
    {
      const uint16_t* qrow = a.q + ((int64_t)b * R + row0 + n) * kDqk + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    }
    float m_ref = kNegBig, lsum = 0.f;
    f32x4_t o[MBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // this lane's DMA source row for block blk of the piece (blocks past the end and
    // out-of-range table entries read an in-bounds row; they are not used)
    auto source = [&](int blk) -> const uint16_t* {
      const int bb = min(blk, nblk - 1);
      const int tok0 = tb + kBlock * bb;
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.page_shift, a.num_pages, b, tok0);
      if (base < 0) base = 0;
      const int t = min(ld_token, te - 1 - tok0);
      return a.kv + (base + t) * kDqk + 8 * g;
    };
    // Wave w moves block w / 2 of the step, 64-B chunk steps 9 (w % 2) .. 9 (w % 2) + 8 (each
    // load: 16 tokens x 4 chunks of 16 B).
    auto issue_step = [&](int k) {
      const int j = wave >> 1, jj0 = LOADS * (wave & 1);
      const uint16_t* src = source(k * SB + j) + 32 * jj0;
      const uint32_t dst = (uint32_t)(uintptr_t)(lds + (k % SLOTS) * (SB * kBlockBytes) + j * kBlockBytes + 1024 * jj0);
      if (stream)
        dma_group_share<true>(src, dst);
      else
        dma_group_share<false>(src, dst);
    };
    // S^T = K Q^T for one 16-token block: this lane's 4 scaled scores (log2 units)
    auto scores = [&](LDS_AS uint8_t* st, int nvalid, float* s) {
      f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      LDS_AS const uint8_t* kp = st + k_lane;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        f32x4_t& acc = (kk & 1) ? acc2 : sacc;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lds_ld128(kp + 1024 * kk)), qf[kk],
                                                      acc, 0, 0, 0);
      }
      sacc += acc2;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (4 * g + i < nvalid) ? sacc[i] * a.scale_log2 : -INFINITY;
    };
    // O^T += V^T P^T for this wave's columns over the step's 32 tokens.  The contraction
    // index k = 8g + j is token 4g + j of the first block (j < 4) or 4g + j - 4 of the
    // second: what the S^T layout leaves in this lane and what one transpose read per
    // block delivers (an unused block's V^T columns were zeroed in the slot).
    // p = exp2(s - m_ref) goes in as bf16 (bf16 output) or as bf16 hi + lo, two MFMAs
    // (fp32 output, about 16 mantissa bits).
    auto accumulate = [&](LDS_AS uint8_t* st, const float (&s)[8]) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        lsum += p[i];
      }
      u32x4_t ph, pl;
      if constexpr (OUT_F32) {
        const u32x4_t q0 = split_hi_lo(p[0], p[1], p[2], p[3]), q1 = split_hi_lo(p[4], p[5], p[6], p[7]);
        ph = u32x4_t{q0[0], q0[1], q1[0], q1[1]};
        pl = u32x4_t{q0[2], q0[3], q1[2], q1[3]};
      } else {
        ph = u32x4_t{bf16x2_rne(p[0], p[1]), bf16x2_rne(p[2], p[3]), bf16x2_rne(p[4], p[5]), bf16x2_rne(p[6], p[7])};
      }
      LDS_AS const uint8_t* vp0 = st + v_lane;
      LDS_AS const uint8_t* vp1 = st + kBlockBytes + v_lane;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const u32x2_t va = lds_tr16(vp0 + 512 * mb), vb = lds_tr16(vp1 + 512 * mb);
        const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, u32x4_t{va[0], va[1], vb[0], vb[1]});
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, __builtin_bit_cast(bf16x8_t, ph), o[mb], 0, 0, 0);
        if constexpr (OUT_F32)
          o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, __builtin_bit_cast(bf16x8_t, pl), o[mb], 0, 0, 0);
      }
    };

    // TS: O^T += V^T P^T over the 16 tokens of one block (sb), as in the 16-row kernel:
    // bf16 weights on a 16x16x16 MFMA (bf16 output) or hi + lo on a 16x16x32 MFMA against
    // V^T repeated twice (fp32 output)
    auto accumulate1 = [&](LDS_AS const uint8_t* sb, const float (&s)[8]) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        lsum += p[i];
      }
      LDS_AS const uint8_t* vp = sb + v_lane;
      if constexpr (OUT_F32) {
        const u32x4_t pp = split_hi_lo(p[0], p[1], p[2], p[3]);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
          const u32x2_t va = lds_tr16(vp + 512 * mb);
          o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u32x4_t{va[0], va[1], va[0], va[1]}),
                                                          __builtin_bit_cast(bf16x8_t, pp), o[mb], 0, 0, 0);
        }
      } else {
        const i16x4_t pp = __builtin_bit_cast(i16x4_t, u32x2_t{bf16x2_rne(p[0], p[1]), bf16x2_rne(p[2], p[3])});
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
          o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, lds_tr16(vp + 512 * mb)), pp,
                                                            o[mb], 0, 0, 0);
      }
    };

    for (int k = 0; k < SLOTS - 1 && k < steps; ++k) issue_step(k);
    int k = 0;
    while (k < steps) {
      float s[8], mx = 0.f;
      bool rescale = false, use0 = false, use1 = false;
      LDS_AS uint8_t* st = lds;
      for (; k < steps; ++k) {
        if (steps - 1 - k >= 2) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
        } else if (steps - 1 - k == 1) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        // step k is in LDS (each wave waited for its own DMA) and every wave is done with
        // step k-1, whose slot the prefetch below overwrites.  A bare s_barrier: a fenced
        // __syncthreads would also wait for the prefetches still in flight.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k + SLOTS - 1 < steps) issue_step(k + SLOTS - 1);
        const int blk0 = k * SB;
        const int tok0 = tb + kBlock * blk0, tok1 = tok0 + kBlock;
        use0 = blk0 < nblk;
        use1 = blk0 + 1 < nblk;
        if (use0 && kv_row_of(block_table, a.bt_stride, a.page_size, a.page_shift, a.num_pages, b, tok0) < 0) use0 = false;
        if (use1 && kv_row_of(block_table, a.bt_stride, a.page_size, a.page_shift, a.num_pages, b, tok1) < 0) use1 = false;
        if ((blk0 < nblk && !use0) || (blk0 + 1 < nblk && !use1)) {
          if (lane == 0) __hip_atomic_fetch_or(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if constexpr (TS) {
          // this wave's block of the step; an unused block is skipped (no other wave of the
          // row group reads it)
          if (!(th ? use1 : use0)) continue;
          st = lds + (k % SLOTS) * (SB * kBlockBytes) + th * kBlockBytes;
          scores(st, lim - (th ? tok1 : tok0), s);
          mx = wave_max_over_groups(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
          if (__any(mx > m_ref + kRescaleSlack)) {
            rescale = true;
            break;
          }
          accumulate1(st, s);
          continue;
        }
        if (!use0 && !use1) continue;
        st = lds + (k % SLOTS) * (SB * kBlockBytes);
        if (!use0 || !use1) {
          // rare: one block of the step is past the end or has an out-of-range table entry
          // (its rows may hold anything): zero that block's 512 V^T columns, 2 chunks of 16
          // tokens x 16 B per 16-column block (every wave reads them all and writes the same
          // zeros first)
          LDS_AS uint8_t* zb = st + (use0 ? kBlockBytes : 0);
          for (int u = lane; u < 32 * MBW; u += 64) *(LDS_AS u32x4_t*)(zb + 16 * u) = u32x4_t{0u, 0u, 0u, 0u};
        }
        scores(st, use0 ? lim - tok0 : 0, s);
        scores(st + kBlockBytes, use1 ? lim - tok1 : 0, s + 4);
        float m8 = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, s[i]);
        mx = wave_max_over_groups(m8);
        if (__any(mx > m_ref + kRescaleSlack)) {
          rescale = true;
          break;
        }
        accumulate(st, s);
      }
      if (!rescale) break;
      // rare path: the running max grew past the slack; move the reference and rescale
      {
        const bool need = mx > m_ref + kRescaleSlack;
        const float f = need ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
        m_ref = need ? mx : m_ref;
        lsum *= f;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) o[mb] *= f;
        if constexpr (TS)
          accumulate1(st, s);
        else
          accumulate(st, s);
        ++k;
      }
    }

    if constexpr (TS) {
      // ---- merge the two waves of each row group (rows 16 rg + n; wave rg took the first
      // block of every step, wave rg + 2 the second) and write
      const float lrow = wave_sum_over_groups(lsum);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();                                // slots no longer read
      asm volatile("" ::: "memory");
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
        for (int mb = 0; mb < MBW; ++mb) *(LDS_AS f32x4_t*)(my + 16 * mb) = o[mb];
      }
      __syncthreads();
      const int rr = threadIdx.x >> 3, dseg = threadIdx.x & 7;     // row of the 32, 4-column piece
      const int w0 = rr >> 4, w1 = w0 + 2, rn = rr & 15;
      const float m0 = sm_m[w0 * 16 + rn], m1 = sm_m[w1 * 16 + rn];
      const float M = fmaxf(m0, m1);
      const float f0 = (m0 <= kNegBig) ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
      const float f1 = (m1 <= kNegBig) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
      const float L = f0 * sm_l[w0 * 16 + rn] + f1 * sm_l[w1 * 16 + rn];
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      const int grow = rgroup * 16 * RG + rr;
#pragma unroll
      for (int j = 0; j < kDv / 32; ++j) {
        const int d = 4 * dseg + 32 * j;
        const f32x4_t v = (f0 * *(LDS_AS const f32x4_t*)(buf + (w0 * 16 + rn) * kMergeStride + d) +
                           f1 * *(LDS_AS const f32x4_t*)(buf + (w1 * 16 + rn) * kMergeStride + d)) * inv;
        if (slot < 0) {
          const int64_t off = ((int64_t)b * R + grow) * kDv + d;
          if (OUT_F32) {
            *(f32x4_t*)((float*)a.out + off) = v;
          } else {
            u32x2_t pkd;
            pkd[0] = bf16x2_rne(v[0], v[1]);
            pkd[1] = bf16x2_rne(v[2], v[3]);
            *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
          }
        } else {
          *(f32x4_t*)(a.part_o + ((int64_t)slot * R + grow) * kDv + d) = v;
        }
      }
      if (dseg == 0) {
        const float lse = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
        if (slot < 0) {
          if (a.lse) a.lse[(int64_t)b * R + grow] = lse;
        } else {
          a.part_lse[(int64_t)slot * R + grow] = lse;
        }
      }
    } else {
    // ---- write: every wave holds its 16 rows complete
      const float l = wave_sum_over_groups(lsum);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int grow = row0 + n;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int d = 16 * mb + 4 * g;
        const f32x4_t v = o[mb] * inv;
        if (slot < 0) {
          const int64_t off = ((int64_t)b * R + grow) * kDv + d;
          if (OUT_F32) {
            *(f32x4_t*)((float*)a.out + off) = v;
          } else {
            u32x2_t pkd;
            pkd[0] = bf16x2_rne(v[0], v[1]);
            pkd[1] = bf16x2_rne(v[2], v[3]);
            *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
          }
        } else {
          *(f32x4_t*)(a.part_o + ((int64_t)slot * R + grow) * kDv + d) = v;
        }
      }
      if (g == 0) {
        const float lse = l > 0.f ? (m_ref + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
        if (slot < 0) {
          if (a.lse) a.lse[(int64_t)b * R + grow] = lse;
        } else {
          a.part_lse[(int64_t)slot * R + grow] = lse;
        }
      }
    }
    // the next piece's prefetch reuses the slots: every wave must be done reading them
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
}

// Log-sum-exp merge of one batch of partial results into a running (M, L, acc): with
// M' = max(M, l_u), acc and L are scaled by e^(M - M') and each partial u adds
// w_u = e^(l_u - M') times its o (and w_u to L).  Partials with l = -inf (no tokens) add
// nothing.
__device__ __forceinline__ void merge_batch(const float (&l)[kMergeBatch], const f32x4_t (&v)[kMergeBatch],
                                            float& M, float& L, f32x4_t& acc) {
  float mb = M;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) mb = fmaxf(mb, l[u]);
  if (mb == -INFINITY) return;
  const float f = M > -INFINITY ? __expf(M - mb) : 0.f;
  L *= f;
  acc *= f;
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const float w = (l[u] > -INFINITY) ? __expf(l[u] - mb) : 0.f;
    L += w;
    acc += w * v[u];
  }
  M = mb;
}

// Merge of split sequences.  One work-group per (sequence, 16 query rows, 64
// output columns): thread (r, q) merges row r, columns 4q..4q+3 of the slice over
// all of the sequence's partial results, so every partial byte is read once and
// all loads of a thread are independent.
constexpr int kMergeCols = 64;
template <bool OUT_F32>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
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
  }
  const int r = rg * 16 + (threadIdx.x >> 4);
  const int d = cg * kMergeCols + 4 * (threadIdx.x & 15);
  const float* lse_col = a.part_lse + (int64_t)s0 * R + r;                 // stride R per slot
  const float* o_col = a.part_o + ((int64_t)s0 * R + r) * kDv + d;         // stride R*512 per slot
  // one pass: kMergeBatch partial results (their lse and 4 columns of o) are loaded at once,
  // so the loads of a batch overlap; the running max moves per batch
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; s += kMergeBatch) {
    float l[kMergeBatch];
    f32x4_t v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool in = s + u < ns;
      l[u] = in ? lse_col[(int64_t)(s + u) * R] : -INFINITY;
      v[u] = in ? *(const f32x4_t*)(o_col + (int64_t)(s + u) * R * kDv) : f32x4_t{0.f, 0.f, 0.f, 0.f};
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


template <bool DEV>
void launch_split(const DecodeArgs& a, bool out_fp32, int grid, hipStream_t s) {
  if (a.kv_fp8) {
    if (out_fp32)
      hipLaunchKernelGGL((split_decode_kernel<true, true, DEV>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((split_decode_kernel<false, true, DEV>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    if (out_fp32)
      hipLaunchKernelGGL((split_decode_kernel<true, false, DEV>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((split_decode_kernel<false, false, DEV>), dim3(grid), dim3(kThreads), 0, s, a);
  }
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
  if (device_schedule || a.kv_fp8) {
    if (rows_per_group != 16) return (int)hipErrorInvalidValue;
    if (device_schedule)
      launch_split<true>(a, out_fp32, grid, s);
    else
      launch_split<false>(a, out_fp32, grid, s);
  } else if (rows_per_group == 16) {
    launch_split<false>(a, out_fp32, grid, s);
  } else if (rows_per_group == 32) {
    if (out_fp32)
      hipLaunchKernelGGL((group_decode_kernel<2, true, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((group_decode_kernel<2, false, true>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if (rows_per_group == 64) {
    if (out_fp32)
      hipLaunchKernelGGL((group_decode_kernel<4, true, false>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((group_decode_kernel<4, false, false>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
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

int launch_merge(const MergeArgs& a, bool out_fp32, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int grid = a.num_merges * (a.rows / 16) * (kDv / kMergeCols);
  if (out_fp32)
    hipLaunchKernelGGL((merge_kernel<true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<false>), dim3(grid), dim3(256), 0, s, a);
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

}  // namespace mla
