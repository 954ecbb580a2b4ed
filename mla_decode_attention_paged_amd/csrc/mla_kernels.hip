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
constexpr int kF8WaveBytes = 2 * kF8Stage + kBlockBytes;       // two fp8 stages + one bf16 stage
constexpr int kSmemFp8 = kWaves * kF8WaveBytes;                // 157,696
constexpr int kLoadsPerBlock = kBlockBytes / (64 * 16);      // 18 DMA loads per wave per block
// Cache policy of the KV-cache DMA loads.  With one row group every KV row is read by one
// work-group only, and the loads carry the non-temporal bit (`nt`): on MI355X a
// global->LDS stream with `nt` runs at ~6.9 TB/s against ~6.1 TB/s without it (read-only
// stream of 1.2 GB, 256 work-groups).  With several row groups the work-groups of one token
// range re-read it through their XCD's L2, and default-policy loads keep it there.
constexpr int kKvLoadStream = 2;   // nt
constexpr int kKvLoadReuse = 0;
constexpr float kRescaleSlack = 8.0f;              // lazy rescale threshold (log2 units)
constexpr int kMinBlocks = kWaves;                 // device schedule: fewest blocks per work-group
constexpr int kMergeBatch = 8;                     // partial results read at a time when merging
constexpr float kNegBig = -1.0e30f;                // running-max start value (finite)
constexpr int kMergeStride = kDv + 4;              // floats per row in the merge buffer

// Chunk-major block layout of the grouped kernel (16-B units): chunk c of token t sits at
// 16 * c + (t ^ ((c & 1) * kSwz)).
constexpr int kSwz = 8;

// Physical row of logical token t of sequence b (the page walk).  Returns -1
// when the block-table entry is outside [0, num_pages).
template <class TablePtr>
__device__ __forceinline__ int64_t kv_row_of(TablePtr block_table, int bt_stride, int page_size,
                                             int num_pages, int b, int t) {
  const int page = block_table[(int64_t)b * bt_stride + t / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + (t % page_size);
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

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }


// Batched LDS reads in inline asm, each block waiting for its own reads before it
// ends.  Outputs are early-clobber: a read can return while later reads of the same
// block still need their address registers, so no output may share one.  Issuing a batch back to back (instead of one read, one wait) keeps many
// LDS requests in flight; doing it in asm also keeps the compiler from adding a
// wait for the in-flight global->LDS prefetch of the other stage before every read.
#define MLA_O4(b, s) "i"(b), "i"(b + s), "i"(b + 2 * s), "i"(b + 3 * s)

// 16-B reads at p + OFF + 1024*i
template <int OFF>
__device__ __forceinline__ void lds_read_b128x6(u32x4_t (&r)[6], LDS_AS const uint8_t* p) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:%7\n\tds_read_b128 %1, %6 offset:%8\n\tds_read_b128 %2, %6 offset:%9\n\t"
      "ds_read_b128 %3, %6 offset:%10\n\tds_read_b128 %4, %6 offset:%11\n\tds_read_b128 %5, %6 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(p), MLA_O4(OFF, 1024), "i"(OFF + 4096), "i"(OFF + 5120)
      : "memory");
}
// transpose reads (4 tokens x 16 columns per 16 lanes) at p + OFF + 512*i
template <int OFF>
__device__ __forceinline__ void lds_read_tr8(u32x2_t (&r)[8], LDS_AS const uint8_t* p) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%9\n\tds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\tds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\tds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%15\n\tds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(p), MLA_O4(OFF, 512), MLA_O4(OFF + 2048, 512)
      : "memory");
}
// Row-major block layout of the split kernel (16-B units): chunk c of token t sits at
// 128 * (c / 8) + 8 * t + ((c % 8) ^ row_swz(t)).  One DMA instruction fills 8 tokens x
// 8 chunks (128 contiguous bytes of each row); the xor spreads the K reads (16 tokens x
// one chunk) and the V^T transpose reads over all LDS banks.
__device__ __forceinline__ int row_swz(int t) { return ((t & 2) << 1) | ((t & 4) >> 1); }

// K operand reads of the row-major layout: k-steps K0..K0+8, even ones at pe + 2048*(kk/2),
// odd ones at po + 2048*(kk/2)
template <int K0>
__device__ __forceinline__ void lds_read_k9(u32x4_t (&r)[9], LDS_AS const uint8_t* pe, LDS_AS const uint8_t* po) {
  if constexpr (K0 == 0) {
    asm volatile(
        "ds_read_b128 %0, %9 offset:0\n\tds_read_b128 %1, %10 offset:0\n\tds_read_b128 %2, %9 offset:2048\n\t"
        "ds_read_b128 %3, %10 offset:2048\n\tds_read_b128 %4, %9 offset:4096\n\tds_read_b128 %5, %10 offset:4096\n\t"
        "ds_read_b128 %6, %9 offset:6144\n\tds_read_b128 %7, %10 offset:6144\n\tds_read_b128 %8, %9 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8])
        : "v"(pe), "v"(po)
        : "memory");
  } else {
    static_assert(K0 == 9, "two halves");
    asm volatile(
        "ds_read_b128 %0, %10 offset:8192\n\tds_read_b128 %1, %9 offset:10240\n\tds_read_b128 %2, %10 offset:10240\n\t"
        "ds_read_b128 %3, %9 offset:12288\n\tds_read_b128 %4, %10 offset:12288\n\tds_read_b128 %5, %9 offset:14336\n\t"
        "ds_read_b128 %6, %10 offset:14336\n\tds_read_b128 %7, %9 offset:16384\n\tds_read_b128 %8, %10 offset:16384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8])
        : "v"(pe), "v"(po)
        : "memory");
  }
}
// V^T transpose reads of the row-major layout: column blocks mb = 16*H .. 16*H+15, block mb at
// p[mb % 4] + 2048 * (mb / 4)
template <int H>
__device__ __forceinline__ void lds_read_v16(u32x2_t (&r)[16], LDS_AS const uint8_t* const (&p)[4]) {
  constexpr int B = 8192 * H;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%20\n\tds_read_b64_tr_b16 %1, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%20\n\tds_read_b64_tr_b16 %3, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:%21\n\tds_read_b64_tr_b16 %5, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:%21\n\tds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%22\n\tds_read_b64_tr_b16 %9, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%22\n\tds_read_b64_tr_b16 %11, %19 offset:%22\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:%23\n\tds_read_b64_tr_b16 %13, %17 offset:%23\n\t"
      "ds_read_b64_tr_b16 %14, %18 offset:%23\n\tds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), MLA_O4(B, 2048)
      : "memory");
}

// Reads of one lane's share of an fp8 stage: 128 latent bytes at pl, 32 rope bytes at pr
// and a 4-byte group scale at ps.
__device__ __forceinline__ void lds_read_f8(u32x4_t (&lat)[8], u32x4_t (&rope)[2], uint32_t& scale,
                                            LDS_AS const uint8_t* pl, LDS_AS const uint8_t* pr,
                                            LDS_AS const uint8_t* ps) {
  asm volatile(
      "ds_read_b128 %0, %11 offset:0\n\tds_read_b128 %1, %11 offset:16\n\tds_read_b128 %2, %11 offset:32\n\t"
      "ds_read_b128 %3, %11 offset:48\n\tds_read_b128 %4, %11 offset:64\n\tds_read_b128 %5, %11 offset:80\n\t"
      "ds_read_b128 %6, %11 offset:96\n\tds_read_b128 %7, %11 offset:112\n\t"
      "ds_read_b128 %8, %12 offset:0\n\tds_read_b128 %9, %12 offset:16\n\tds_read_b32 %10, %13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lat[0]), "=&v"(lat[1]), "=&v"(lat[2]), "=&v"(lat[3]), "=&v"(lat[4]), "=&v"(lat[5]),
        "=&v"(lat[6]), "=&v"(lat[7]), "=&v"(rope[0]), "=&v"(rope[1]), "=&v"(scale)
      : "v"(pl), "v"(pr), "v"(ps)
      : "memory");
}
// Writes of one lane's converted share into the bf16 stage: chunk m of the first 8 at
// w[m], of the second 8 at w[m] + 2048, the two rope chunks at r0 and r1.
__device__ __forceinline__ void lds_write_bf16(LDS_AS uint8_t* const (&w)[8], LDS_AS uint8_t* r0, LDS_AS uint8_t* r1,
                                               const u32x4_t (&c)[16], const u32x4_t (&rope)[2]) {
  asm volatile(
      "ds_write_b128 %0, %10\n\tds_write_b128 %1, %11\n\tds_write_b128 %2, %12\n\tds_write_b128 %3, %13\n\t"
      "ds_write_b128 %4, %14\n\tds_write_b128 %5, %15\n\tds_write_b128 %6, %16\n\tds_write_b128 %7, %17\n\t"
      "ds_write_b128 %0, %18 offset:2048\n\tds_write_b128 %1, %19 offset:2048\n\t"
      "ds_write_b128 %2, %20 offset:2048\n\tds_write_b128 %3, %21 offset:2048\n\t"
      "ds_write_b128 %4, %22 offset:2048\n\tds_write_b128 %5, %23 offset:2048\n\t"
      "ds_write_b128 %6, %24 offset:2048\n\tds_write_b128 %7, %25 offset:2048\n\t"
      "ds_write_b128 %8, %26\n\tds_write_b128 %9, %27\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(r0), "v"(r1),
        "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(c[4]), "v"(c[5]), "v"(c[6]), "v"(c[7]),
        "v"(c[8]), "v"(c[9]), "v"(c[10]), "v"(c[11]), "v"(c[12]), "v"(c[13]), "v"(c[14]), "v"(c[15]),
        "v"(rope[0]), "v"(rope[1])
      : "memory");
}

// Split-decode kernel: 16 query rows per work-group (R = 16 * row groups).  FP8: the cache
// rows are 656-byte fp8 rows (see kF8Row); each block goes through a small fp8 stage and
// is widened into one bf16 stage in the row-major layout, where the bf16 path reads it.
// DEV: no host schedule; the work-groups cut the batch's blocks among themselves from the
// device cache_seqlens and combine split sequences in the same launch (see below).
template <bool OUT_F32, bool FP8, bool DEV>
__global__ void __launch_bounds__(kThreads, 1) split_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[FP8 ? kSmemFp8 : kSmemBytes];
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

  // bf16: two DMA stages; FP8: two fp8 DMA stages and one bf16 stage the blocks are widened into
  LDS_AS uint8_t* stage0 = FP8 ? lds + wave * kF8WaveBytes : lds + (wave * kStages + 0) * kBlockBytes;
  LDS_AS uint8_t* stage1 = FP8 ? stage0 + kF8Stage : lds + (wave * kStages + 1) * kBlockBytes;
  LDS_AS uint8_t* const cstage = FP8 ? stage0 + 2 * kF8Stage : nullptr;
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

    // query rows as MFMA B operands (Q^T): lane (n, g) holds row n, columns 32*kk + 8*g .. +8
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
      const uint16_t* p[2];   // bf16: this lane's source for even / odd instructions
      const uint8_t* row0;    // FP8: the block's first row
      int last;               // FP8: index of the block's last valid row
    };
    auto source = [&](int k, bool& ok) -> Src {
      const int tok0 = tb + kBlock * blk_of(k);
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.num_pages, b, tok0);
      ok = base >= 0;
      if (!ok) base = 0;
      const int last = te - 1 - tok0;
      Src r{};
      if constexpr (FP8) {
        r.row0 = kv8 + base * kF8Row;
        r.last = last;
      } else {
        r.p[0] = a.kv + (base + min(ld_tok0, last)) * kDqk + ld_col0;
        r.p[1] = a.kv + (base + min(ld_tok1, last)) * kDqk + ld_col1;
      }
      return r;
    };
    // The DMA loads of a block into a stage.  bf16: 18 instructions of 1 KB, each 128 B of 8
    // rows (chunk block j/2).  FP8: the 656 16-B units of the 16 rows in row order, 64 per
    // instruction (the 11th moves the last 16).
    auto issue = [&](const Src& src, LDS_AS uint8_t* stage) {
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < kF8Loads; ++j) {
          const int u = 64 * j + lane;
          if (j + 1 < kF8Loads || u < kF8Units) {
            const int t = u / (kF8Row / 16), c = u - t * (kF8Row / 16);
            GLB_AS void* gp = (GLB_AS void*)(src.row0 + min(t, src.last) * kF8Row + 16 * c);
            if (stream)
              __builtin_amdgcn_global_load_lds(gp, (LDS_AS void*)(stage + 1024 * j), 16, 0, kKvLoadStream);
            else
              __builtin_amdgcn_global_load_lds(gp, (LDS_AS void*)(stage + 1024 * j), 16, 0, kKvLoadReuse);
          }
        }
      } else if (stream) {
#pragma unroll
        for (int j = 0; j < kLoadsPerBlock; ++j)
          __builtin_amdgcn_global_load_lds((GLB_AS void*)(src.p[j & 1] + 64 * (j >> 1)),
                                           (LDS_AS void*)(stage + 1024 * j), 16, 0, kKvLoadStream);
      } else {
#pragma unroll
        for (int j = 0; j < kLoadsPerBlock; ++j)
          __builtin_amdgcn_global_load_lds((GLB_AS void*)(src.p[j & 1] + 64 * (j >> 1)),
                                           (LDS_AS void*)(stage + 1024 * j), 16, 0, kKvLoadReuse);
      }
    };
    // FP8: widen an fp8 stage into the bf16 stage.  Lane (t = lane % 16, q = lane / 16)
    // converts latent columns [128q, 128q + 128) of token t (one group scale, which the
    // conversion applies through its exponent) and copies rope chunks 2q, 2q + 1.
    auto widen = [&](LDS_AS const uint8_t* f8, LDS_AS uint8_t* dst) {
      const int t = lane & 15, q = lane >> 4;
      u32x4_t lat[8], rope[2];
      uint32_t scale_bits;
      lds_read_f8(lat, rope, scale_bits, f8 + t * kF8Row + 128 * q, f8 + t * kF8Row + 512 + 32 * q,
                  f8 + t * kF8Row + 640 + 4 * q);
      const float scale = __uint_as_float(scale_bits);
      u32x4_t c[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t x = lat[i][2 * h + w];
            c[2 * i + h][2 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, scale, false));
            c[2 * i + h][2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, scale, true));
          }
        }
      }
      // chunk m of this lane's 16 is column chunk 16q + m of token t: unit
      // 128 * (2q + m / 8) + 8t + ((m % 8) ^ row_swz(t)); rope chunk 64 + 2q + i likewise
      const int sw = row_swz(t);
      LDS_AS uint8_t* w[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) w[m] = dst + 16 * (256 * q + 8 * t + (m ^ sw));
      LDS_AS uint8_t* r0 = dst + 16 * (1024 + 8 * t + ((2 * q) ^ sw));
      LDS_AS uint8_t* r1 = dst + 16 * (1024 + 8 * t + ((2 * q + 1) ^ sw));
      lds_write_bf16(w, r0, r1, c, rope);
    };
    // Every LDS read of a block first (K for S^T, then all of V^T into registers); then the
    // stage is refilled with the block after next (`ns`, if `nx`) while S^T, the softmax
    // and O^T += V^T P^T are still being computed.
    auto scores = [&](LDS_AS uint8_t* st, f32x4_t& sacc, u32x2_t (&vf0)[16], u32x2_t (&vf1)[16], const Src& ns,
                      bool nx) {
      f32x4_t acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto mma = [&](const u32x4_t* kf, int kk0) {
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          f32x4_t& acc = ((kk0 + i) & 1) ? acc2 : sacc;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[i]), qf[kk0 + i], acc, 0, 0, 0);
        }
      };
      u32x4_t kf[9];
      lds_read_k9<0>(kf, st + k_even, st + k_odd);
      mma(kf, 0);
      lds_read_k9<9>(kf, st + k_even, st + k_odd);
      LDS_AS const uint8_t* const vp[4] = {st + v_base[0], st + v_base[1], st + v_base[2], st + v_base[3]};
      lds_read_v16<0>(vf0, vp);                // columns 0..255
      lds_read_v16<1>(vf1, vp);                // columns 256..511
      if (!FP8 && nx) issue(ns, st);
      mma(kf, 9);
      sacc += acc2;
    };
    // O^T += V^T P^T for one block, p = exp2(s - m_ref).  p is split into two bf16
    // terms, p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), and both go through the
    // MFMA, so the weights carry ~16 mantissa bits instead of bf16's 8; the running
    // sum l takes p in fp32.
    auto accumulate = [&](const float (&s)[4], const u32x2_t (&vf0)[16], const u32x2_t (&vf1)[16]) {
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);
        hb[i] = bf16_rne(p);
        lb[i] = bf16_rne(p - bf16_bits_to_float(hb[i]));
        lsum += p;
      }
      const i16x4_t ph = i16x4_t{(short)hb[0], (short)hb[1], (short)hb[2], (short)hb[3]};
      const i16x4_t pl = i16x4_t{(short)lb[0], (short)lb[1], (short)lb[2], (short)lb[3]};
      auto pv = [&](const u32x2_t (&vf)[16], int mb0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const i16x4_t v = __builtin_bit_cast(i16x4_t, vf[i]);
          o[mb0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, ph, o[mb0 + i], 0, 0, 0);
          o[mb0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pl, o[mb0 + i], 0, 0, 0);
        }
      };
      pv(vf0, 0);
      pv(vf1, 16);
    };

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
          if constexpr (FP8)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kF8Loads) : "memory");
          else
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
        if constexpr (FP8) {
          widen(st, cstage);
          if (nx) issue(nsrc, st);
          scores(cstage, sacc, vf0, vf1, nsrc, false);
        } else {
          scores(st, sacc, vf0, vf1, nsrc, nx);
        }
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
            pkd[0] = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
            pkd[1] = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
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

// Grouped split-decode kernel for 16 * RG query rows per work-group.  The four
// waves consume the same KV stream: wave (rg, dh) owns query rows 16*rg..16*rg+15
// and output columns [512*dh/DH, 512*(dh+1)/DH) with DH = 4 / RG.  Each step is
// 32 tokens (two 16-token blocks); the work-group keeps four step slots in LDS
// (three steps in flight), filled by global->LDS DMA split evenly over the waves
// (9 loads each per step), and moves from step to step behind one barrier that
// publishes the step's data and frees the slot read in the previous step.  Every
// wave computes S^T for its rows over all 576 columns (the waves of a row group
// repeat it) and O^T += V^T P^T for its columns on 16x16x32 MFMA with K = 32 tokens.
template <int RG, bool OUT_F32>
__global__ void __launch_bounds__(kThreads, 1) group_decode_kernel(DecodeArgs a) {
  constexpr int DH = kWaves / RG;                       // column parts
  constexpr int SB = 2;                                 // blocks per step
  constexpr int SLOTS = kWaves * kStages / SB;          // step slots (4)
  constexpr int LOADS = kLoadsPerBlock * SB / kWaves;   // DMA instructions per wave and step (9)
  constexpr int MBW = kVBlocks / DH;                    // 16-column output blocks per wave
  static_assert(LOADS * kWaves == kLoadsPerBlock * SB && MBW % 8 == 0, "layout");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int rg = wave / DH, dh = wave % DH;

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
  const int mb0 = dh * MBW;

  const int k_lane = (g * 16 + (n ^ ((g & 1) * kSwz))) * 16;
  const int e = n >> 2, qq = n & 3;
  const int v_lane = ((qq >> 1) * 16 + ((4 * g + e) ^ ((qq >> 1) * kSwz))) * 16 + (qq & 1) * 8 + mb0 * 512;
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
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.num_pages, b, tok0);
      if (base < 0) base = 0;
      const int t = min(ld_token, te - 1 - tok0);
      return a.kv + (base + t) * kDqk + 8 * g;
    };
    auto issue_step = [&](int k) {
      LDS_AS uint8_t* dst = lds + (k % SLOTS) * (SB * kBlockBytes);
      const uint16_t* src0 = source(k * SB);
      const uint16_t* src1 = source(k * SB + 1);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int I = wave + kWaves * i;                // the step's I-th DMA (of 36)
        const int j = I / kLoadsPerBlock, jj = I % kLoadsPerBlock;
        const uint16_t* src = j ? src1 : src0;
        if (stream)
          __builtin_amdgcn_global_load_lds((GLB_AS void*)(src + 32 * jj),
                                           (LDS_AS void*)(dst + j * kBlockBytes + 1024 * jj), 16, 0, kKvLoadStream);
        else
          __builtin_amdgcn_global_load_lds((GLB_AS void*)(src + 32 * jj),
                                           (LDS_AS void*)(dst + j * kBlockBytes + 1024 * jj), 16, 0, kKvLoadReuse);
      }
    };
    // S^T = K Q^T for one 16-token block: this lane's 4 scaled scores (log2 units)
    auto scores = [&](LDS_AS uint8_t* st, int nvalid, float* s) {
      f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, acc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u32x4_t kf[6];
      LDS_AS const uint8_t* kp = st + k_lane;
      auto mma = [&](int kk0) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          f32x4_t& acc = (i & 1) ? acc2 : sacc;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[i]), qf[kk0 + i], acc, 0, 0, 0);
        }
      };
      lds_read_b128x6<0>(kf, kp);
      mma(0);
      lds_read_b128x6<6144>(kf, kp);
      mma(6);
      lds_read_b128x6<12288>(kf, kp);
      mma(12);
      sacc += acc2;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (4 * g + i < nvalid) ? sacc[i] * a.scale_log2 : -INFINITY;
    };
    // O^T += V^T P^T for this wave's columns over the step's 32 tokens.  The contraction
    // index k = 8g + j is token 4g + j of the first block (j < 4) or 4g + j - 4 of the
    // second: what the S^T layout leaves in this lane and what one transpose read per
    // block delivers.  A block that is not used contributes a zero V^T half.
    // p = exp2(s - m_ref) goes in as bf16 hi + lo (about 16 mantissa bits).
    auto accumulate = [&](LDS_AS uint8_t* st, const float (&s)[8], bool use0, bool use1) {
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);
        hb[i] = bf16_rne(p);
        lb[i] = bf16_rne(p - bf16_bits_to_float(hb[i]));
        lsum += p;
      }
      u32x4_t ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = hb[2 * i] | (hb[2 * i + 1] << 16);
        pl[i] = lb[2 * i] | (lb[2 * i + 1] << 16);
      }
      const uint32_t keep0 = use0 ? 0xFFFFFFFFu : 0u, keep1 = use1 ? 0xFFFFFFFFu : 0u;
      LDS_AS const uint8_t* vp0 = st + v_lane;
      LDS_AS const uint8_t* vp1 = st + kBlockBytes + v_lane;
      u32x2_t va[8], vb[8];
      auto pv = [&](int mbl) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u32x4_t v;
          v[0] = va[i][0] & keep0;
          v[1] = va[i][1] & keep0;
          v[2] = vb[i][0] & keep1;
          v[3] = vb[i][1] & keep1;
          const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, v);
          o[mbl + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, __builtin_bit_cast(bf16x8_t, ph), o[mbl + i], 0,
                                                               0, 0);
          o[mbl + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, __builtin_bit_cast(bf16x8_t, pl), o[mbl + i], 0,
                                                               0, 0);
        }
      };
      lds_read_tr8<0>(va, vp0);
      lds_read_tr8<0>(vb, vp1);
      pv(0);
      if constexpr (MBW > 8) {
        lds_read_tr8<4096>(va, vp0);
        lds_read_tr8<4096>(vb, vp1);
        pv(8);
      }
      if constexpr (MBW > 16) {
        lds_read_tr8<8192>(va, vp0);
        lds_read_tr8<8192>(vb, vp1);
        pv(16);
        lds_read_tr8<12288>(va, vp0);
        lds_read_tr8<12288>(vb, vp1);
        pv(24);
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
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k + SLOTS - 1 < steps) issue_step(k + SLOTS - 1);
        const int blk0 = k * SB;
        const int tok0 = tb + kBlock * blk0, tok1 = tok0 + kBlock;
        use0 = blk0 < nblk;
        use1 = blk0 + 1 < nblk;
        if (use0 && kv_row_of(block_table, a.bt_stride, a.page_size, a.num_pages, b, tok0) < 0) use0 = false;
        if (use1 && kv_row_of(block_table, a.bt_stride, a.page_size, a.num_pages, b, tok1) < 0) use1 = false;
        if ((blk0 < nblk && !use0) || (blk0 + 1 < nblk && !use1)) {
          if (lane == 0) __hip_atomic_fetch_or(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (!use0 && !use1) continue;
        st = lds + (k % SLOTS) * (SB * kBlockBytes);
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
        accumulate(st, s, use0, use1);
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
        accumulate(st, s, use0, use1);
        ++k;
      }
    }

    // ---- write: every wave holds complete rows for its columns (all waves of a row
    // group agree on m_ref and l, having computed the same scores)
    {
      const float l = wave_sum_over_groups(lsum);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int grow = row0 + n;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int d = 16 * (mb0 + mb) + 4 * g;
        const f32x4_t v = o[mb] * inv;
        if (slot < 0) {
          const int64_t off = ((int64_t)b * R + grow) * kDv + d;
          if (OUT_F32) {
            *(f32x4_t*)((float*)a.out + off) = v;
          } else {
            u32x2_t pkd;
            pkd[0] = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
            pkd[1] = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
            *(u32x2_t*)((uint16_t*)a.out + off) = pkd;
          }
        } else {
          *(f32x4_t*)(a.part_o + ((int64_t)slot * R + grow) * kDv + d) = v;
        }
      }
      if (dh == 0 && g == 0) {
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
  const CST_AS int32_t* merges = as_const(a.merges);
  const int b = merges[4 * item + 0];
  const int s0 = merges[4 * item + 1];
  const int ns = merges[4 * item + 2];
  const int r = rg * 16 + (threadIdx.x >> 4);
  const int d = cg * kMergeCols + 4 * (threadIdx.x & 15);
  const float* lse_col = a.part_lse + (int64_t)s0 * R + r;                 // stride R per slot
  const float* o_col = a.part_o + ((int64_t)s0 * R + r) * kDv + d;         // stride R*512 per slot
  // loads are issued kMergeBatch at a time so their latencies overlap
  float M = -INFINITY;
  for (int s = 0; s < ns; s += kMergeBatch) {
    float l[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) l[u] = (s + u < ns) ? lse_col[(int64_t)(s + u) * R] : -INFINITY;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) M = fmaxf(M, l[u]);
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < ns; s += kMergeBatch) {
      float l[kMergeBatch];
      f32x4_t v[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const bool in = s + u < ns;
        l[u] = in ? lse_col[(int64_t)(s + u) * R] : -INFINITY;
        v[u] = in ? *(const f32x4_t*)(o_col + (int64_t)(s + u) * R * kDv) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = (l[u] > -INFINITY) ? __expf(l[u] - M) : 0.f;
        L += w;
        acc += w * v[u];
      }
    }
  }
  const f32x4_t v = acc * (L > 0.f ? 1.0f / L : 0.f);
  const int64_t off = ((int64_t)b * R + r) * kDv + d;
  if (OUT_F32) {
    *(f32x4_t*)((float*)a.out + off) = v;
  } else {
    u32x2_t pkd;
    pkd[0] = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    pkd[1] = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
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
  float M = -INFINITY;
  for (int w0 = wf; w0 <= wl; w0 += kMergeBatch) {
    float l[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int sl = w0 + u <= wl ? slot_of(w0 + u) : -1;
      l[u] = sl >= 0 ? a.part_lse[(int64_t)sl * R + r] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) M = fmaxf(M, l[u]);
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M > -INFINITY) {
    for (int w0 = wf; w0 <= wl; w0 += kMergeBatch) {
      float l[kMergeBatch];
      f32x4_t v[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int sl = w0 + u <= wl ? slot_of(w0 + u) : -1;
        l[u] = sl >= 0 ? a.part_lse[(int64_t)sl * R + r] : -INFINITY;
        v[u] = sl >= 0 ? *(const f32x4_t*)(a.part_o + ((int64_t)sl * R + r) * kDv + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = (l[u] > -INFINITY) ? __expf(l[u] - M) : 0.f;
        L += w;
        acc += w * v[u];
      }
    }
  }
  const f32x4_t v = acc * (L > 0.f ? 1.0f / L : 0.f);
  const int64_t off = ((int64_t)b * R + r) * kDv + d;
  if (OUT_F32) {
    *(f32x4_t*)((float*)a.out + off) = v;
  } else {
    u32x2_t pkd;
    pkd[0] = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    pkd[1] = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
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
  const int64_t row = kv_row_of(block_table, bt_stride, page_size, num_pages, seq, t);
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
      hipLaunchKernelGGL((group_decode_kernel<2, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((group_decode_kernel<2, false>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if (rows_per_group == 64) {
    if (out_fp32)
      hipLaunchKernelGGL((group_decode_kernel<4, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((group_decode_kernel<4, false>), dim3(grid), dim3(kThreads), 0, s, a);
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
