// Kernels of the steps on either side of the absorbed decode: the query
// up-projection with rotary embedding, the append of new cache rows, and the
// value up-projection of the decode's latent output.
//
// Low-rank joint KV compression (FlashMLA-on-Ascend post, the section on the
// compression principle and its computation flow): head h's keys and values are
// K_h = C W_UK[h], V_h = C W_UV[h] for the shared latent rows C.  Folding W_UK
// into the query and applying W_UV after attention gives the 576-wide absorbed
// rows the decode reads (FlashMLA-ETAP summary, "Implementation details").
//
// Weights are stored so both MFMA operands are plain 16-byte loads along the
// contraction dimension: W_UK as [H, 512, 128] (latent column, nope column),
// W_UV as [H, 128, 512] (output column, latent column).
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNope = 128;       // per-head query columns before absorption
constexpr int kRope = 64;        // rotary columns
constexpr int kVout = 128;       // per-head output columns after the value up-projection
constexpr int kLayerThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float64 -> bf16, round to nearest even, in one rounding: truncate to float32
// and keep a sticky bit in the last place (round to odd, exact for any target
// with at least two fewer significand bits), then round that to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const float f = __double2float_rz(d);
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) u |= 1u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Rotary embedding of one pair (x[2i], x[2i+1]) at position pos: rotation by
// pos * base^(-2i/64), evaluated in float64 and rounded once to bf16.
__device__ __forceinline__ uint32_t rope_pair_bf16x2(uint32_t packed, int pos, int i, double base) {
  const double x0 = bf16_to_f32(packed & 0xFFFFu), x1 = bf16_to_f32(packed >> 16);
  const double ang = (double)pos * pow(base, -2.0 * i / kRope);
  double s, c;
  sincos(ang, &s, &c);
  const uint32_t y0 = f64_to_bf16_rne(x0 * c - x1 * s);
  const uint32_t y1 = f64_to_bf16_rne(x0 * s + x1 * c);
  return y0 | (y1 << 16);
}

// Nearest OCP E4M3 code of y (|y| <= 448), ties to the even code, sign from y's sign bit.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                 // |y| < 2^-6: subnormal codes n * 2^-9 (n = 8 is 2^-6)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                               // rebias the exponent (127 -> 7), keep 3 fraction bits
    const uint32_t t = a - (120u << 23);
    code = t >> 20;
    const uint32_t rem = t & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
  }
  return code | ((u >> 24) & 0x80u);
}

// Smallest e >= -126 with amax <= 448 * 2^e (0 when amax == 0): amax = m 2^E, m in [0.5, 1),
// and 448 = 0.875 * 2^9, so e = E - 9, plus one when m > 0.875.
__device__ __forceinline__ int fp8_group_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  const int e = E - 9 + (m > 0.875f ? 1 : 0);
  return e < -126 ? -126 : e;
}

// ---------------------------------------------------------------------------------------------
// Query preparation.  grid (512 / 64, H), 256 threads.  Wave w of work-group (x, h) computes
// latent columns e0 = 64x + 16w .. e0 + 15 of head h for every token as the MFMA tile
// C[e][n] = sum_d W_UK[h][e][d] q_nope[n][h][d]; then the work-group rotates rope pairs
// 4x .. 4x + 3 of head h for every token.
__global__ __launch_bounds__(kLayerThreads) void q_absorb_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ w_uk,
    const int32_t* __restrict__ positions, int ntok, int H, double base, uint16_t* __restrict__ q_out) {
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int e0 = 64 * blockIdx.x + 16 * wave;

  bf16x8_t af[kNope / 32];   // A: lane (m, g) holds W_UK[h][e0 + m][32 kk + 8 g .. + 8]
  {
    const uint16_t* wrow = w_uk + ((int64_t)h * kDv + e0 + m) * kNope + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kNope / 32; ++kk) af[kk] = *(const bf16x8_t*)(wrow + 32 * kk);
  }
  for (int n0 = 0; n0 < ntok; n0 += 16) {
    const int n = n0 + m;
    bf16x8_t bq[kNope / 32];   // B: lane (n, g) holds q_nope[n][h][32 kk + 8 g .. + 8]
    if (n < ntok) {
      const uint16_t* qrow = q_nope + ((int64_t)n * H + h) * kNope + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kNope / 32; ++kk) bq[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < kNope / 32; ++kk) bq[kk] = bf16x8_t{};
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kNope / 32; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk], bq[kk], acc, 0, 0, 0);
    if (n < ntok) {   // lane (n, g) holds latent columns e0 + 4g .. + 4 of token n
      u32x2_t pk;
      pk[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
      pk[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
      *(u32x2_t*)(q_out + ((int64_t)n * H + h) * kDqk + e0 + 4 * g) = pk;
    }
  }
  for (int t = threadIdx.x; t < ntok * 4; t += kLayerThreads) {
    const int n = t >> 2, i = 4 * blockIdx.x + (t & 3);
    const uint32_t x = *(const uint32_t*)(q_pe + ((int64_t)n * H + h) * kRope + 2 * i);
    *(uint32_t*)(q_out + ((int64_t)n * H + h) * kDqk + kDv + 2 * i) = rope_pair_bf16x2(x, positions[n], i, base);
  }
}

// ---------------------------------------------------------------------------------------------
// Cache append.  One wave per new token n = b * q_len + s, 4 per work-group.  The row of
// position positions[n] is row positions[n] % P of page block_table[b][positions[n] / P];
// a position outside [0, max_pages_per_seq * P) or a page outside [0, num_pages) writes
// nothing and sets bit 1 of *status (when status is not NULL).
template <bool FP8>
__global__ __launch_bounds__(kLayerThreads) void kv_append_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ block_table, int ntok, int q_len, int bt_stride, int page_size, int num_pages,
    int max_pos, double base, uint8_t* __restrict__ kv, int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * (kLayerThreads / 64) + (threadIdx.x >> 6);
  if (n >= ntok) return;
  const int b = n / q_len;
  const int pos = positions[n];
  int64_t row = -1;
  if (pos >= 0 && pos < max_pos) {
    const int page = block_table[(int64_t)b * bt_stride + pos / page_size];
    if (page >= 0 && page < num_pages) row = (int64_t)page * page_size + pos % page_size;
  }
  if (row < 0) {
    if (lane == 0 && status) __hip_atomic_fetch_or(status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // lane j: latent columns 8j .. 8j + 7; lanes 0..31 also rope pair j
  const u32x4_t lat = *(const u32x4_t*)(c_kv + (int64_t)n * kDv + 8 * lane);
  uint32_t pe = 0;
  if (lane < kRope / 2) pe = rope_pair_bf16x2(*(const uint32_t*)(k_pe + (int64_t)n * kRope + 2 * lane), pos, lane, base);
  if constexpr (!FP8) {
    uint8_t* dst = kv + row * kRowBytesBf16;
    *(u32x4_t*)(dst + 16 * lane) = lat;
    if (lane < kRope / 2) *(uint32_t*)(dst + 2 * kDv + 4 * lane) = pe;
  } else {
    uint8_t* dst = kv + row * kRowBytesFp8;
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_to_f32(lat[k] & 0xFFFFu);
      x[2 * k + 1] = bf16_to_f32(lat[k] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    // group of 128 columns = 16 consecutive lanes
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
    const int e = fp8_group_exponent(amax);
    u32x2_t codes = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) codes[k >> 2] |= e4m3_code(ldexpf(x[k], -e)) << (8 * (k & 3));
    *(u32x2_t*)(dst + 8 * lane) = codes;
    if (lane < kRope / 2) *(uint32_t*)(dst + kDv + 4 * lane) = pe;
    if ((lane & 15) == 0) *(float*)(dst + kDv + 2 * kRope + 4 * (lane >> 4)) = ldexpf(1.f, e);
  }
}

// ---------------------------------------------------------------------------------------------
// Output projection.  grid (128 / 16, H), 256 threads.  Work-group (x, h) computes output
// columns v0 = 16x .. v0 + 15 of head h for every token, C[v][n] = sum_e W_UV[h][v][e]
// lat[n][h][e]; wave w takes latent columns 128w .. 128w + 127 and the four partial tiles
// are added through LDS.  A float32 input is fed to the bf16 MFMA as hi + lo, hi = bf16(x),
// lo = bf16(x - hi), which keeps about 16 significant bits of it.
template <bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(kLayerThreads) void out_absorb_kernel(
    const void* __restrict__ lat_v, const uint16_t* __restrict__ w_uv, int ntok, int H, void* __restrict__ out_v) {
  constexpr int kSteps = kDv / 4 / 32;   // 4 MFMA k-steps per wave
  __shared__ f32x4_t red[kLayerThreads / 64 - 1][64];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int v0 = 16 * blockIdx.x;
  const int c0 = 128 * wave + 8 * g;   // this lane's first latent column in k-step 0

  bf16x8_t af[kSteps];   // A: lane (m, g) holds W_UV[h][v0 + m][c0 + 32 kk .. + 8]
  {
    const uint16_t* wrow = w_uv + ((int64_t)h * kVout + v0 + m) * kDv + c0;
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) af[kk] = *(const bf16x8_t*)(wrow + 32 * kk);
  }
  for (int n0 = 0; n0 < ntok; n0 += 16) {
    const int n = n0 + m;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (IN_F32) {
      const float* src = (const float*)lat_v + ((int64_t)n * H + h) * kDv + c0;
#pragma unroll
      for (int kk = 0; kk < kSteps; ++kk) {
        f32x4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (n < ntok) {
          x0 = *(const f32x4_t*)(src + 32 * kk);
          x1 = *(const f32x4_t*)(src + 32 * kk + 4);
        }
        u32x4_t hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = k < 2 ? x0[2 * k] : x1[2 * k - 4], b = k < 2 ? x0[2 * k + 1] : x1[2 * k - 3];
          const uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b);
          hi[k] = ha | (hb << 16);
          lo[k] = f32_to_bf16_rne(a - bf16_to_f32(ha)) | (f32_to_bf16_rne(b - bf16_to_f32(hb)) << 16);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk], __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk], __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
      }
    } else {
      const uint16_t* src = (const uint16_t*)lat_v + ((int64_t)n * H + h) * kDv + c0;
#pragma unroll
      for (int kk = 0; kk < kSteps; ++kk) {
        const bf16x8_t bq = n < ntok ? *(const bf16x8_t*)(src + 32 * kk) : bf16x8_t{};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk], bq, acc, 0, 0, 0);
      }
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kLayerThreads / 64 - 1; ++w) acc += red[w][lane];
      if (n < ntok) {   // lane (n, g) holds output columns v0 + 4g .. + 4 of token n
        const int64_t o = ((int64_t)n * H + h) * kVout + v0 + 4 * g;
        if constexpr (OUT_F32) {
          *(f32x4_t*)((float*)out_v + o) = acc;
        } else {
          u32x2_t pk;
          pk[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
          pk[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
          *(u32x2_t*)((uint16_t*)out_v + o) = pk;
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

int launch_q_absorb(const LayerArgs& a, void* stream_v) {
  const hipStream_t stream = (hipStream_t)stream_v;
  const int ntok = a.batch * a.q_len;
  hipLaunchKernelGGL(q_absorb_kernel, dim3(kDv / 64, a.num_heads), dim3(kLayerThreads), 0, stream,
                     (const uint16_t*)a.q_nope, (const uint16_t*)a.q_pe, (const uint16_t*)a.w_uk, a.positions,
                     ntok, a.num_heads, (double)a.rope_base, (uint16_t*)a.q_out);
  return (int)hipGetLastError();
}

int launch_kv_append(const LayerArgs& a, void* stream_v) {
  const hipStream_t stream = (hipStream_t)stream_v;
  const int ntok = a.batch * a.q_len;
  const dim3 grid((ntok + kLayerThreads / 64 - 1) / (kLayerThreads / 64));
  const int max_pos = a.max_pages_per_seq * a.page_size;
  if (a.kv_fp8)
    hipLaunchKernelGGL(kv_append_kernel<true>, grid, dim3(kLayerThreads), 0, stream, (const uint16_t*)a.c_kv,
                       (const uint16_t*)a.k_pe, a.positions, a.block_table, ntok, a.q_len, a.max_pages_per_seq,
                       a.page_size, a.num_pages, max_pos, (double)a.rope_base, (uint8_t*)a.kv_cache, a.status);
  else
    hipLaunchKernelGGL(kv_append_kernel<false>, grid, dim3(kLayerThreads), 0, stream, (const uint16_t*)a.c_kv,
                       (const uint16_t*)a.k_pe, a.positions, a.block_table, ntok, a.q_len, a.max_pages_per_seq,
                       a.page_size, a.num_pages, max_pos, (double)a.rope_base, (uint8_t*)a.kv_cache, a.status);
  return (int)hipGetLastError();
}

int launch_out_absorb(const LayerArgs& a, bool in_f32, bool out_f32, void* stream_v) {
  const hipStream_t stream = (hipStream_t)stream_v;
  const int ntok = a.batch * a.q_len;
  const dim3 grid(kVout / 16, a.num_heads), block(kLayerThreads);
  if (in_f32 && out_f32)
    hipLaunchKernelGGL((out_absorb_kernel<true, true>), grid, block, 0, stream, a.out_latent, (const uint16_t*)a.w_uv,
                       ntok, a.num_heads, a.o);
  else if (in_f32)
    hipLaunchKernelGGL((out_absorb_kernel<true, false>), grid, block, 0, stream, a.out_latent,
                       (const uint16_t*)a.w_uv, ntok, a.num_heads, a.o);
  else if (out_f32)
    hipLaunchKernelGGL((out_absorb_kernel<false, true>), grid, block, 0, stream, a.out_latent,
                       (const uint16_t*)a.w_uv, ntok, a.num_heads, a.o);
  else
    hipLaunchKernelGGL((out_absorb_kernel<false, false>), grid, block, 0, stream, a.out_latent,
                       (const uint16_t*)a.w_uv, ntok, a.num_heads, a.o);
  return (int)hipGetLastError();
}

}  // namespace mla
