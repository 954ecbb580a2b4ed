// gfx950 kernels for paged MLA decode: split decode, merge of split results,
// and a debug gather that shares the decode kernel's page walk.
//
// Split-decode kernel, one work-group (4 waves) per piece list from the planner.
// Each wave streams its own 16-token KV blocks (blocks w, w+4, w+8, ... of a
// piece) through a private two-stage LDS ring filled by 16-byte
// global->LDS DMA loads, and keeps its own online-softmax state.  Per block it
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
constexpr int kLoadsPerBlock = kBlockBytes / (64 * 16);      // 18 DMA loads per wave per block
constexpr float kRescaleSlack = 8.0f;              // lazy rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;                // running-max start value (finite)
constexpr int kMergeStride = kDv + 4;              // floats per row in the merge buffer

#ifndef MLA_PROGRESSIVE_REFILL
#define MLA_PROGRESSIVE_REFILL 1   // refill a stage part by part as its bytes are consumed
#endif
#ifndef MLA_CONTIG_BLOCKS
#define MLA_CONTIG_BLOCKS 0        // 0: wave w takes blocks w, w+4, ...; 1: a contiguous quarter
#endif

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
// ends.  Issuing a batch back to back (instead of one read, one wait) keeps many
// LDS requests in flight; doing it in asm also keeps the compiler from adding a
// wait for the in-flight global->LDS prefetch of the other stage before every read.
#define MLA_RD128(i, off) "ds_read_b128 %" #i ", %9 offset:" #off "\n\t"
#define MLA_RDTR(i, off) "ds_read_b64_tr_b16 %" #i ", %16 offset:" #off "\n\t"

// Nine 16-B reads at p + 1024*i (i = 0..8) and at p + 9216 + 1024*i.
__device__ __forceinline__ void lds_read_k_lo(u32x4_t (&r)[9], LDS_AS const uint8_t* p) {
  asm volatile(MLA_RD128(0, 0) MLA_RD128(1, 1024) MLA_RD128(2, 2048) MLA_RD128(3, 3072) MLA_RD128(4, 4096)
               MLA_RD128(5, 5120) MLA_RD128(6, 6144) MLA_RD128(7, 7168) MLA_RD128(8, 8192) "s_waitcnt lgkmcnt(0)"
               : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
                 "=v"(r[8])
               : "v"(p)
               : "memory");
}
__device__ __forceinline__ void lds_read_k_hi(u32x4_t (&r)[9], LDS_AS const uint8_t* p) {
  asm volatile(MLA_RD128(0, 9216) MLA_RD128(1, 10240) MLA_RD128(2, 11264) MLA_RD128(3, 12288) MLA_RD128(4, 13312)
               MLA_RD128(5, 14336) MLA_RD128(6, 15360) MLA_RD128(7, 16384) MLA_RD128(8, 17408)
               "s_waitcnt lgkmcnt(0)"
               : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
                 "=v"(r[8])
               : "v"(p)
               : "memory");
}
// Sixteen transpose reads at p + 512*i (i = 0..15) and at p + 8192 + 512*i.
__device__ __forceinline__ void lds_read_vt_lo(u32x2_t (&r)[16], LDS_AS const uint8_t* p) {
  asm volatile(MLA_RDTR(0, 0) MLA_RDTR(1, 512) MLA_RDTR(2, 1024) MLA_RDTR(3, 1536) MLA_RDTR(4, 2048)
               MLA_RDTR(5, 2560) MLA_RDTR(6, 3072) MLA_RDTR(7, 3584) MLA_RDTR(8, 4096) MLA_RDTR(9, 4608)
               MLA_RDTR(10, 5120) MLA_RDTR(11, 5632) MLA_RDTR(12, 6144) MLA_RDTR(13, 6656) MLA_RDTR(14, 7168)
               MLA_RDTR(15, 7680) "s_waitcnt lgkmcnt(0)"
               : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
                 "=v"(r[8]), "=v"(r[9]), "=v"(r[10]), "=v"(r[11]), "=v"(r[12]), "=v"(r[13]), "=v"(r[14]),
                 "=v"(r[15])
               : "v"(p)
               : "memory");
}
__device__ __forceinline__ void lds_read_vt_hi(u32x2_t (&r)[16], LDS_AS const uint8_t* p) {
  asm volatile(MLA_RDTR(0, 8192) MLA_RDTR(1, 8704) MLA_RDTR(2, 9216) MLA_RDTR(3, 9728) MLA_RDTR(4, 10240)
               MLA_RDTR(5, 10752) MLA_RDTR(6, 11264) MLA_RDTR(7, 11776) MLA_RDTR(8, 12288) MLA_RDTR(9, 12800)
               MLA_RDTR(10, 13312) MLA_RDTR(11, 13824) MLA_RDTR(12, 14336) MLA_RDTR(13, 14848)
               MLA_RDTR(14, 15360) MLA_RDTR(15, 15872) "s_waitcnt lgkmcnt(0)"
               : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
                 "=v"(r[8]), "=v"(r[9]), "=v"(r[10]), "=v"(r[11]), "=v"(r[12]), "=v"(r[13]), "=v"(r[14]),
                 "=v"(r[15])
               : "v"(p)
               : "memory");
}

template <bool OUT_F32>
__global__ void __launch_bounds__(kThreads, 1) split_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
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

  // LDS block layout (16-B units): position = chunk*16 + (token ^ ((chunk & 1) << 2)),
  // chunk = 16-B column chunk 0..71, token 0..15.  K-operand reads are then 1 KB
  // contiguous and the V^T transpose reads touch all banks once per 16 lanes.
  const int k_lane = (g * 16 + (n ^ ((g & 1) << 2))) * 16;
  const int e = n >> 2, qq = n & 3;
  const int v_lane = ((qq >> 1) * 16 + ((4 * g + e) ^ ((qq >> 1) << 2))) * 16 + (qq & 1) * 8;
  const int ld_token = n ^ ((g & 1) << 2);    // token this lane fetches for chunk 4*j + g

  LDS_AS uint8_t* stage0 = lds + (wave * kStages + 0) * kBlockBytes;
  LDS_AS uint8_t* stage1 = lds + (wave * kStages + 1) * kBlockBytes;

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
#if MLA_CONTIG_BLOCKS
    const int blk_first = (wave * nblk) / kWaves;
    const int my_n = ((wave + 1) * nblk) / kWaves - blk_first;
    auto blk_of = [&](int k) { return blk_first + k; };
#else
    const int my_n = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
    auto blk_of = [&](int k) { return wave + kWaves * k; };
#endif

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

    // Source row of this lane for the DMA of the wave's k-th block; `ok` is false for an
    // out-of-range table entry (then page 0 is read, in bounds, and the block is skipped).
    auto source = [&](int k, bool& ok) -> const uint16_t* {
      const int tok0 = tb + kBlock * blk_of(k);
      int64_t base = kv_row_of(block_table, a.bt_stride, a.page_size, a.num_pages, b, tok0);
      ok = base >= 0;
      if (!ok) base = 0;
      const int t = min(ld_token, te - 1 - tok0);   // rows past the end re-read the last valid row
      return a.kv + (base + t) * kDqk + 8 * g;
    };
    // DMA loads j0..j1-1 (1 KB each: 16-B column chunks 4j..4j+3 of the 16 rows) into a stage
    auto issue = [&](const uint16_t* src, LDS_AS uint8_t* stage, int j0, int j1) {
#pragma unroll
      for (int j = j0; j < j1; ++j)
        __builtin_amdgcn_global_load_lds((GLB_AS void*)(src + 32 * j), (LDS_AS void*)(stage + 1024 * j), 16, 0, 0);
    };
    // O^T += V^T P^T for one block, p = exp2(s - m_ref).  p is split into two bf16
    // terms, p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), and both go through the
    // MFMA, so the weights carry ~16 mantissa bits instead of bf16's 8; the running
    // sum l takes p in fp32.  As each half of V^T has been read, the matching part of
    // the stage is refilled with the block after next (`nsrc`, if any).
    auto accumulate = [&](LDS_AS uint8_t* st, const float (&s)[4], const uint16_t* nsrc) {
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
      u32x2_t vf[16];
      lds_read_vt_lo(vf, st + v_lane);           // columns 0..255 = stage bytes [0, 8 KB)
#if MLA_PROGRESSIVE_REFILL
      if (nsrc) issue(nsrc, st, 0, 8);
#endif
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        const i16x4_t v = __builtin_bit_cast(i16x4_t, vf[mb]);
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, ph, o[mb], 0, 0, 0);
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pl, o[mb], 0, 0, 0);
      }
      lds_read_vt_hi(vf, st + v_lane);           // columns 256..511 = stage bytes [8 KB, 16 KB)
#if MLA_PROGRESSIVE_REFILL
      if (nsrc) issue(nsrc, st, 8, 16);
#else
      if (nsrc) issue(nsrc, st, 0, kLoadsPerBlock);
#endif
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        const i16x4_t v = __builtin_bit_cast(i16x4_t, vf[mb]);
        o[16 + mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, ph, o[16 + mb], 0, 0, 0);
        o[16 + mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pl, o[16 + mb], 0, 0, 0);
      }
    };

    bool ok0 = true, ok1 = true;   // table entry of the block now in each stage was in range
    if (my_n > 0) issue(source(0, ok0), stage0, 0, kLoadsPerBlock);
    if (my_n > 1) issue(source(1, ok1), stage1, 0, kLoadsPerBlock);

    int k = 0;
    while (k < my_n) {
      float s[4], mx = 0.f;
      bool rescale = false;
      const uint16_t* nsrc = nullptr;
      // hot loop: o is only touched by MFMA here
      for (; k < my_n; ++k) {
        LDS_AS uint8_t* st = (k & 1) ? stage1 : stage0;
        bool nok = true;
        nsrc = (k + 2 < my_n) ? source(k + 2, nok) : nullptr;
        if (k + 1 < my_n) {
          asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const bool ok = (k & 1) ? ok1 : ok0;
        if (k & 1) ok1 = nok; else ok0 = nok;   // the stage's next occupant
        if (!ok) {
          if (lane == 0) __hip_atomic_fetch_or(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (nsrc) issue(nsrc, st, 0, kLoadsPerBlock);
          continue;
        }
        const int nvalid = te - (tb + kBlock * blk_of(k));   // >= 1
        // S^T = K Q^T: 16 tokens x 16 rows, lane holds tokens 4g..4g+3 of row n
        f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, sacc2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        {
          u32x4_t kf[9];
          lds_read_k_lo(kf, st + k_lane);
#pragma unroll
          for (int kk = 0; kk < 9; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]), qf[kk], sacc, 0, 0, 0);
          lds_read_k_hi(kf, st + k_lane);
#if MLA_PROGRESSIVE_REFILL
          if (nsrc) issue(nsrc, st, 16, kLoadsPerBlock);   // rope columns: stage bytes [16 KB, 18 KB)
#endif
#pragma unroll
          for (int kk = 0; kk < 9; ++kk)
            sacc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]), qf[9 + kk], sacc2, 0,
                                                            0, 0);
        }
        sacc += sacc2;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = (4 * g + i < nvalid) ? sacc[i] * a.scale_log2 : -INFINITY;
        mx = wave_max_over_groups(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        if (__any(mx > m_ref + kRescaleSlack)) {
          rescale = true;
          break;
        }
        accumulate(st, s, nsrc);
      }
      if (!rescale) break;
      // rare path: the running max grew past the slack; move the reference and rescale
      {
        LDS_AS uint8_t* st = (k & 1) ? stage1 : stage0;
        const bool need = mx > m_ref + kRescaleSlack;
        const float f = need ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
        m_ref = need ? mx : m_ref;
        lsum *= f;
#pragma unroll
        for (int mb = 0; mb < kVBlocks; ++mb) o[mb] *= f;
        accumulate(st, s, nsrc);
        ++k;
      }
    }

    // ---- merge the four waves' states and write
    const float lrow = wave_sum_over_groups(lsum);
    __syncthreads();
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
    {
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
  }
}

// Merge of split sequences.  One work-group per (sequence, 16 query rows, 64
// output columns): thread (r, q) merges row r, columns 4q..4q+3 of the slice over
// all of the sequence's partial results, so every partial byte is read once and
// all loads of a thread are independent.
constexpr int kMergeCols = 64;
constexpr int kMergeBatch = 8;
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

// Debug gather: one thread per 16-B chunk of a sequence's logical rows.
__global__ void __launch_bounds__(256) gather_kernel(const uint16_t* kv, const int32_t* block_table, uint16_t* rows_out,
                                                     int32_t seq, int32_t length, int64_t row_offset,
                                                     int32_t page_size, int32_t bt_stride, int32_t num_pages) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(idx / (kDqk / 8));
  const int c = (int)(idx % (kDqk / 8));
  if (t >= length) return;
  const int64_t row = kv_row_of(block_table, bt_stride, page_size, num_pages, seq, t);
  if (row < 0) return;
  *(u32x4_t*)(rows_out + (row_offset + t) * kDqk + 8 * c) = *(const u32x4_t*)(kv + row * kDqk + 8 * c);
}

}  // namespace

int launch_decode(const DecodeArgs& a, int rows_per_group, bool out_fp32, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (rows_per_group != 16) return (int)hipErrorInvalidValue;
  if (out_fp32)
    hipLaunchKernelGGL((split_decode_kernel<true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((split_decode_kernel<false>), dim3(grid), dim3(kThreads), 0, s, a);
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

int launch_gather(const uint16_t* kv, const int32_t* block_table, uint16_t* rows_out, int32_t seq, int32_t length,
                  int64_t row_offset, int32_t page_size, int32_t bt_stride, int32_t num_pages, void* stream) {
  const int64_t chunks = (int64_t)length * (kDqk / 8);
  const int grid = (int)((chunks + 255) / 256);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, kv, block_table, rows_out, seq,
                     length, row_offset, page_size, bt_stride, num_pages);
  return (int)hipGetLastError();
}

const char* hip_error_string(int code) { return hipGetErrorString((hipError_t)code); }

}  // namespace mla
