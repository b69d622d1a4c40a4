// Block quantisation of GEMM operands to OCP e4m3.
//
// Blockwise FP8 shares one scale among a block of values ("Prime
// Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster", section
// "Precision and hardware support").  Three block shapes are used:
//   rows:    1 x 128 along a row (activations and gradients in the forward
//            and data-gradient GEMMs, blocks along their K dimension);
//   weights: 128 x 128 tiles of one expert's matrix;
//   tokens:  128 consecutive rows of one expert's segment x 1 column (both
//            operands of the weight-gradient GEMMs, whose K is the token
//            dimension), the count starting at the expert's first row.
// For a block with largest magnitude amax the scale is s = amax / 448 in
// fp32 (s = 1 for an all-zero block) and each value x becomes the e4m3
// number nearest to the fp32 quotient x / s, ties to even; the GEMMs use
// q * s.  The token-blocked operands are written transposed ([column][row],
// each expert's rows padded with zeros to a multiple of 128) so that every
// GEMM operand is contiguous along its K dimension.
//
// MXFP8 (same section: smaller scaling groups) uses the OCP microscaling
// layout instead: 32 values along each GEMM operand's K share a power-of-two
// scale 2^X stored as an E8M0 byte (X + 127).  X is the smallest integer
// with amax <= 448 * 2^X (the blockwise scale rounded up to a power of two,
// so nothing saturates), at least -127, and 0 for an all-zero block; x / 2^X
// is exact in fp32, so each code is the e4m3 rounding of the exact quotient.
// Rows take 1 x 32 blocks; a weight is encoded twice, 1 x 32 along K for
// the forward and 32 x 1 along N (written transposed) for the data
// gradients; token operands take 32-row blocks inside the same 128-row
// padded runs.  Four consecutive blocks' codes form one 32-bit word, so a
// 128-wide K step of the GEMMs reads one word per row, as with fp32 scales.
//
// The kernels can write the scale words row-major (the layouts of the C
// ABI's quantise entry points) or run-major, [K/128][rows], for the GEMMs:
// there one K step's words for consecutive rows are contiguous.
#include "common.h"
#include "tile.h"

namespace moe {
namespace {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;

// Scale of a block with largest magnitude amax (correctly rounded division).
__device__ __forceinline__ float block_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
}

// v / s as the e4m3 encoding sees it, without a full division per value.
// q = v * rs, with rs the rounded reciprocal of s, lies within 2.5 fp32
// ulps of the rounded quotient: two roundings of relative size 2^-24, plus
// the quotient's own half ulp.  e4m3 keeps three mantissa bits, so its
// rounding decides on the 20 bits below them; unless those bits of q lie
// within 8 ulps of the midpoint pattern 0x80000, q and the rounded quotient
// are on the same side of every e4m3 midpoint, with no tie, and give the
// same code.  Near a midpoint, and below e4m3's normal range (2^-6, where
// its grid is fixed at 2^-9), the exact quotient is taken.
__device__ __forceinline__ float quot_e4m3(float v, float s, float rs) {
  const float q = v * rs;
  const int d = (int)(__float_as_uint(q) & 0xFFFFFu) - 0x80000;
  const bool safe = v == 0.0f || ((d > 8 || d < -8) && fabsf(q) >= 0x1p-6f);
  return safe ? q : __fdiv_rn(v, s);
}

// e4m3 codes of four quotients packed little-endian.  v_cvt_pk_fp8_f32
// rounds to nearest even; the operand is clamped to +-448 first, so values a
// rounding of s pushed just past 448 saturate instead of overflowing.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const float lo = -kE4M3Max, hi = kE4M3Max;
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), v, true);
  return (uint32_t)v;
}

__device__ __forceinline__ void unpack8(const u32x4_t v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// MXFP8 block scale: E8M0 code X + 127 and the exact multiplier 2^-X.
struct MxScale {
  uint32_t code;
  float inv;
};
__device__ __forceinline__ MxScale mx_scale(float amax) {
  const uint32_t u = __float_as_uint(amax);  // amax >= 0
  int X = 0;
  if (u != 0) {
    // amax = m 2^e with m in [1, 2) (subnormals give e = -127, far below the
    // clamp): X = e - 8, plus one when m > 1.75 (448 = 1.75 * 2^8)
    X = (int)(u >> 23) - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    X = X < -127 ? -127 : X;
  }
  return MxScale{(uint32_t)(X + 127), __uint_as_float((uint32_t)(127 - X) << 23)};
}

// Eight values times 2^-X (exact), as eight e4m3 codes.
__device__ __forceinline__ u32x2_t quant8_mx(const float (&f)[8], float inv) {
  u32x2_t q;
  q[0] = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
  q[1] = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
  return q;
}

// Codes of lanes base, base + stride, base + 2 stride, base + 3 stride
// packed little-endian into one word (every lane gets it).
__device__ __forceinline__ uint32_t gather4_codes(uint32_t code, int base, int stride) {
  return (uint32_t)__shfl((int)code, base, kWave) | ((uint32_t)__shfl((int)code, base + stride, kWave) << 8) |
         ((uint32_t)__shfl((int)code, base + 2 * stride, kWave) << 16) |
         ((uint32_t)__shfl((int)code, base + 3 * stride, kWave) << 24);
}

// Eight values divided by s, as eight e4m3 codes.
__device__ __forceinline__ u32x2_t quant8(const float (&f)[8], float s) {
  u32x2_t q;
  const float rs = __fdiv_rn(1.0f, s);
  q[0] = e4m3x4(quot_e4m3(f[0], s, rs), quot_e4m3(f[1], s, rs), quot_e4m3(f[2], s, rs), quot_e4m3(f[3], s, rs));
  q[1] = e4m3x4(quot_e4m3(f[4], s, rs), quot_e4m3(f[5], s, rs), quot_e4m3(f[6], s, rs), quot_e4m3(f[7], s, rs));
  return q;
}

// ---------------------------------------------------------------------------
// Blocks along rows: src [rows, C] (leading dimension ld) -> q [rows, C] and
// one scale word per row and 128 columns: fp32 (1 x 128 blocks) or, MX, the
// E8M0 bytes of four 1 x 32 blocks.  The word of (row r, column block cb)
// sits at s[r * s_row + cb * s_blk]: row-major (C / 128, 1) or run-major
// (1, rows), where one K step's words of consecutive rows are contiguous.
// With row_of (token rows of x or dout), each token row's word goes to the
// k expert-sorted rows row_of[r k + j] instead, run-major over those rows:
// a GEMM that gathers the token rows then reads its words contiguously.
// A 16-lane group handles 128 columns, 8 values a lane.
// ---------------------------------------------------------------------------
template <bool MX>
__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16_t* __restrict__ src, int64_t ld,
                                                        int64_t rows, int C, uint8_t* __restrict__ q,
                                                        void* __restrict__ s, int64_t s_row, int64_t s_blk,
                                                        const int32_t* __restrict__ row_of, int k) {
  const int nbc = C / 128;
  const int64_t nb = rows * nbc;
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sl = threadIdx.x & 15;
  const bool ok = g < nb;
  const int64_t r = ok ? g / nbc : 0;
  const int cb = ok ? (int)(g % nbc) : 0;
  u32x4_t v = {0, 0, 0, 0};
  if (ok) v = *(const u32x4_t*)(src + r * ld + cb * 128 + sl * 8);
  float f[8];
  unpack8(v, f);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  if constexpr (MX) {
    // four lanes per 32-value block
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    const MxScale sc = mx_scale(amax);
    const int lane = threadIdx.x & 63;
    const uint32_t word = gather4_codes(sc.code, lane & ~15, 4);
    if (!ok) return;
    *(u32x2_t*)(q + r * C + cb * 128 + sl * 8) = quant8_mx(f, sc.inv);
    if (sl == 0) {
      if (row_of)
        for (int j = 0; j < k; ++j) ((uint32_t*)s)[(int64_t)row_of[r * k + j] * s_row + cb * s_blk] = word;
      else
        ((uint32_t*)s)[r * s_row + cb * s_blk] = word;
    }
  } else {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const float sc = block_scale(amax);
    if (!ok) return;
    *(u32x2_t*)(q + r * C + cb * 128 + sl * 8) = quant8(f, sc);
    if (sl == 0) {
      if (row_of)
        for (int j = 0; j < k; ++j) ((float*)s)[(int64_t)row_of[r * k + j] * s_row + cb * s_blk] = sc;
      else
        ((float*)s)[r * s_row + cb * s_blk] = sc;
    }
  }
}

// Staged code tiles: 128 rows of 32 words (+1 of padding) in LDS, leaving
// as 16-byte pieces of 128-byte rows.
constexpr int kWS = 33;  // staged code rows: 32 words + 1 of padding

__device__ __forceinline__ void store_code_tile(const uint32_t* tile, uint8_t* dst, int64_t ld) {
  // 128 rows x 128 bytes: chunk c = 16 bytes (4 words) of row c / 8
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = p * 256 + threadIdx.x;
    const int row = c >> 3, w = (c & 7) * 4;
    const uint32_t* src = tile + row * kWS + w;
    *(u32x4_t*)(dst + (int64_t)row * ld + w * 4) = u32x4_t{src[0], src[1], src[2], src[3]};
  }
}

// The 128 x 128 bf16 block at Wb (row stride K elements) as floats: thread
// t gets rows 4 (t % 32) .. +3, columns 16 (t / 32) .. +15.  The block goes
// through LDS (stage: 32 KB) on direct loads that read whole 256-byte rows,
// 16-byte chunk c of row r landing at chunk c ^ ((r / 4) % 16) of its LDS
// row, so that the 32 rows one half-wave reads at a column are spread over
// the banks.  Read straight from memory, each load instruction took 16 bytes
// from each of 32 rows.  Ends with a barrier: stage may be reused at once.
__device__ __forceinline__ void load_block_staged(const bf16_t* Wb, int K, tile::lds_t* stage,
                                                  float (&f)[4][16]) {
  const int t = threadIdx.x, w = tile::wave_id(), l = t & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = w * 8 + i;  // 1 KB of LDS: rows 4q .. 4q+3
    const int row = 4 * q + (l >> 4);
    const int c = (l & 15) ^ ((row >> 2) & 15);
    tile::dma16(Wb + (int64_t)row * K + c * 8, stage + q * 1024);
  }
  tile::wait_vmcnt<0>();
  __syncthreads();
  const int n0 = 4 * (t & 31), c0 = 2 * (t >> 5);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = n0 + j, sw = (row >> 2) & 15;
    const tile::lds_t* r = stage + row * 256;
    float lo[8], hi[8];
    unpack8(*(const __attribute__((address_space(3))) u32x4_t*)(r + ((c0 ^ sw) << 4)), lo);
    unpack8(*(const __attribute__((address_space(3))) u32x4_t*)(r + (((c0 + 1) ^ sw) << 4)), hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[j][i] = lo[i];
      f[j][8 + i] = hi[i];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// 128 x 128 weight blocks of W [E, N, K], written as q [E, N, K] with s [E,
// N/128, K/128] and/or transposed as qt [E, K, N] with st [E, K/128, N/128]
// (either pair may be null).  One work-group per block; thread t holds rows
// 4 (t % 32) .. +3 and columns 16 (t / 32) .. +15 of it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_weight_kernel(const bf16_t* __restrict__ W, int N, int K,
                                                          uint8_t* __restrict__ q, float* __restrict__ s,
                                                          uint8_t* __restrict__ qt,
                                                          float* __restrict__ st) {
  __shared__ float red[4];
  // the staged bf16 block, then the code tiles fcodes [n][32 words] and
  // tcodes [k][32 words]
  __shared__ __attribute__((aligned(16))) uint32_t smem[2 * 128 * kWS];
  uint32_t* const fcodes = smem;
  uint32_t* const tcodes = smem + 128 * kWS;
  const int kb = blockIdx.x, nb = blockIdx.y, e = blockIdx.z;
  const int t = threadIdx.x;
  const int n0 = 4 * (t & 31), k0 = 16 * (t >> 5);
  float f[4][16];
  load_block_staged(W + (int64_t)e * N * K + (int64_t)(nb * 128) * K + kb * 128, K, (tile::lds_t*)smem, f);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[j][i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  const float sc = block_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  const float rsc = __fdiv_rn(1.0f, sc);
  const int nbn = N / 128, nbk = K / 128;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) f[j][i] = quot_e4m3(f[j][i], sc, rsc);
  // q, qt are kernel arguments: every branch on them is uniform
  if (qt) {  // a transposed row gets four consecutive codes from each of 32 lanes
#pragma unroll
    for (int i = 0; i < 16; ++i) tcodes[(k0 + i) * kWS + (n0 >> 2)] = e4m3x4(f[0][i], f[1][i], f[2][i], f[3][i]);
  }
  if (q) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        fcodes[(n0 + j) * kWS + (k0 >> 2) + w] =
            e4m3x4(f[j][4 * w], f[j][4 * w + 1], f[j][4 * w + 2], f[j][4 * w + 3]);
  }
  __syncthreads();
  if (qt) {
    store_code_tile(tcodes, qt + (int64_t)e * K * N + (int64_t)(kb * 128) * N + nb * 128, N);
    if (t == 0) st[((int64_t)e * nbk + kb) * nbn + nb] = sc;
  }
  if (q) {
    store_code_tile(fcodes, q + (int64_t)e * N * K + (int64_t)(nb * 128) * K + kb * 128, K);
    if (t == 0) s[((int64_t)e * nbn + nb) * nbk + kb] = sc;
  }
}

// ---------------------------------------------------------------------------
// MXFP8 weights W [E, N, K], encoded twice from one read: q [E, N, K] with
// 1 x 32 blocks along K and scales s [E, N, K/32], and qt [E, K, N] (the
// transpose) with 1 x 32 blocks along N and scales st [E, K, N/32]; either
// pair may be null (not written).  run_major: the scale words (four codes
// each) are stored [E, K/128, N] and [E, N/128, K] instead, so that the
// words of one 128-wide K step for consecutive rows are contiguous.  One
// work-group per 128 x 128 tile; thread
// t holds rows 4 (t % 32) .. +3 and columns 16 (t / 32) .. +15 of it, so a
// row's 32-column block spans lanes t and t ^ 32 and a column's 32-row
// block spans the 8 lanes t ^ 0..7.  Both code tiles and both scale tiles
// are staged in LDS and leave as 16-byte rows (codes) and 32-bit words (a
// row's or column's four scale bytes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_weight_mx_kernel(const bf16_t* __restrict__ W, int N, int K,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                             uint8_t* __restrict__ qt,
                                                             uint8_t* __restrict__ st, int run_major) {
  // the staged bf16 block, then the code tiles fcodes [n][32 words] and
  // tcodes [k][32 words]
  __shared__ __attribute__((aligned(16))) uint32_t smem[2 * 128 * kWS];
  __shared__ uint32_t fscale[128], tscale[128];  // [n], [k]: 4 bytes each
  uint32_t* const fcodes = smem;
  uint32_t* const tcodes = smem + 128 * kWS;
  const int kb = blockIdx.x, nb = blockIdx.y, e = blockIdx.z;
  const int t = threadIdx.x;
  const int n0 = 4 * (t & 31), k0 = 16 * (t >> 5);
  float f[4][16];
  load_block_staged(W + (int64_t)e * N * K + (int64_t)(nb * 128) * K + kb * 128, K, (tile::lds_t*)smem, f);
  // q, qt are kernel arguments: every branch on them is uniform
  if (q) {  // forward layout: row blocks along K
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(f[j][i]));
      const MxScale rs = mx_scale(fmaxf(a, __shfl_xor(a, 32, kWave)));
#pragma unroll
      for (int w = 0; w < 4; ++w)
        fcodes[(n0 + j) * kWS + (k0 >> 2) + w] =
            e4m3x4(f[j][4 * w] * rs.inv, f[j][4 * w + 1] * rs.inv, f[j][4 * w + 2] * rs.inv,
                   f[j][4 * w + 3] * rs.inv);
      if (((t >> 5) & 1) == 0) ((uint8_t*)fscale)[(n0 + j) * 4 + (t >> 6)] = (uint8_t)rs.code;
    }
  }
  if (qt) {  // transposed layout: column blocks along N, four rows' codes per word
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = fmaxf(fmaxf(fabsf(f[0][i]), fabsf(f[1][i])), fmaxf(fabsf(f[2][i]), fabsf(f[3][i])));
      a = fmaxf(a, __shfl_xor(a, 1, kWave));
      a = fmaxf(a, __shfl_xor(a, 2, kWave));
      a = fmaxf(a, __shfl_xor(a, 4, kWave));
      const MxScale cs = mx_scale(a);
      tcodes[(k0 + i) * kWS + (n0 >> 2)] =
          e4m3x4(f[0][i] * cs.inv, f[1][i] * cs.inv, f[2][i] * cs.inv, f[3][i] * cs.inv);
      if ((t & 7) == 0) ((uint8_t*)tscale)[(k0 + i) * 4 + ((t & 31) >> 3)] = (uint8_t)cs.code;
    }
  }
  __syncthreads();
  if (q) {
    store_code_tile(fcodes, q + (int64_t)e * N * K + (int64_t)(nb * 128) * K + kb * 128, K);
    if (t < 128) {
      const int64_t n = nb * 128 + t;
      const int64_t w = run_major ? ((int64_t)e * (K / 128) + kb) * N + n : ((int64_t)e * N + n) * (K / 128) + kb;
      ((uint32_t*)s)[w] = fscale[t];
    }
  }
  if (qt) {
    store_code_tile(tcodes, qt + (int64_t)e * K * N + (int64_t)(kb * 128) * N + nb * 128, N);
    if (t >= 128) {
      const int k = t - 128;
      const int64_t kk = kb * 128 + k;
      const int64_t w = run_major ? ((int64_t)e * (N / 128) + nb) * K + kk : ((int64_t)e * K + kk) * (N / 128) + nb;
      ((uint32_t*)st)[w] = tscale[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Token blocks, transposed.  Block b (of blk_off[E] in all) is the
// (b - blk_off[e])-th run of 128 rows of expert e's segment; row i of the run
// is src row srow(offsets[e] + 128 * (b - blk_off[e]) + i), with srow(r) =
// src_of[r] / kdiv (token rows of x or dout) or r.  A work-group handles 64
// columns: q[c][128 b + i] = code (0 past the segment) and the scale word
// of (column c, run b) at s[c * s_row + b * s_blk]: the run's fp32 scale or,
// MX, the E8M0 codes of its four 32-row blocks.  Run-major words (s_row = 1,
// s_blk = columns) put the words of one run for consecutive columns side by
// side, as one K step of the weight-gradient GEMMs reads them.
// ---------------------------------------------------------------------------
constexpr int kTokCols = 64;

template <bool MX>
__global__ __launch_bounds__(256) void quant_tok_kernel(const bf16_t* __restrict__ src, int64_t ld,
                                                       const int32_t* __restrict__ src_of, int kdiv,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ blk_off, int E,
                                                       uint8_t* __restrict__ q, int64_t ldq,
                                                       uint32_t* __restrict__ s, int64_t s_row, int64_t s_blk) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 136];  // [row][64 bf16], 136-byte rows
  const int b = blockIdx.x;
  if (b >= blk_off[E]) return;
  int lo = 0, hi = E;  // largest e with blk_off[e] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (blk_off[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int r0 = offsets[e] + (b - blk_off[e]) * 128;
  const int n = min(128, offsets[e + 1] - r0);
  const int c0 = blockIdx.y * kTokCols;
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = (t >> 3) + 32 * p, ch = t & 7;
    u32x4_t v = {0, 0, 0, 0};
    if (i < n) {
      const int64_t sr = src_of ? (int64_t)(src_of[r0 + i] / kdiv) : (int64_t)(r0 + i);
      v = *(const u32x4_t*)(src + sr * ld + c0 + ch * 8);
    }
    u32x2_t* dst = (u32x2_t*)(tile + i * 136 + ch * 16);
    dst[0] = u32x2_t{v[0], v[1]};
    dst[1] = u32x2_t{v[2], v[3]};
  }
  __syncthreads();
  // thread: column pair cp (columns c0 + 2cp, +1), rows 16 rg .. 16 rg + 15
  const int cp = t >> 3, rg = t & 7;
  float f0[16], f1[16];
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = *(const uint32_t*)(tile + (16 * rg + i) * 136 + cp * 4);
    f0[i] = __uint_as_float(w << 16);
    f1[i] = __uint_as_float(w & 0xFFFF0000u);
    a0 = fmaxf(a0, fabsf(f0[i]));
    a1 = fmaxf(a1, fabsf(f1[i]));
  }
  const int c = c0 + 2 * cp;
  u32x4_t q0, q1;
  uint32_t w0, w1;
  if constexpr (MX) {  // a 32-row block spans lanes rg = 2m, 2m + 1
    a0 = fmaxf(a0, __shfl_xor(a0, 1, kWave));
    a1 = fmaxf(a1, __shfl_xor(a1, 1, kWave));
    const MxScale s0 = mx_scale(a0), s1 = mx_scale(a1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q0[w] = e4m3x4(f0[4 * w] * s0.inv, f0[4 * w + 1] * s0.inv, f0[4 * w + 2] * s0.inv, f0[4 * w + 3] * s0.inv);
      q1[w] = e4m3x4(f1[4 * w] * s1.inv, f1[4 * w + 1] * s1.inv, f1[4 * w + 2] * s1.inv, f1[4 * w + 3] * s1.inv);
    }
    const int base = (t & 63) & ~7;
    w0 = gather4_codes(s0.code, base, 2);
    w1 = gather4_codes(s1.code, base, 2);
  } else {
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      a0 = fmaxf(a0, __shfl_xor(a0, off, kWave));
      a1 = fmaxf(a1, __shfl_xor(a1, off, kWave));
    }
    const float s0 = block_scale(a0), s1 = block_scale(a1);
    const float r0 = __fdiv_rn(1.0f, s0), r1 = __fdiv_rn(1.0f, s1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q0[w] = e4m3x4(quot_e4m3(f0[4 * w], s0, r0), quot_e4m3(f0[4 * w + 1], s0, r0),
                     quot_e4m3(f0[4 * w + 2], s0, r0), quot_e4m3(f0[4 * w + 3], s0, r0));
      q1[w] = e4m3x4(quot_e4m3(f1[4 * w], s1, r1), quot_e4m3(f1[4 * w + 1], s1, r1),
                     quot_e4m3(f1[4 * w + 2], s1, r1), quot_e4m3(f1[4 * w + 3], s1, r1));
    }
    w0 = __float_as_uint(s0);
    w1 = __float_as_uint(s1);
  }
  *(u32x4_t*)(q + (int64_t)c * ldq + (int64_t)b * 128 + rg * 16) = q0;
  *(u32x4_t*)(q + (int64_t)(c + 1) * ldq + (int64_t)b * 128 + rg * 16) = q1;
  if (rg == 0) {
    s[(int64_t)c * s_row + (int64_t)b * s_blk] = w0;
    s[(int64_t)(c + 1) * s_row + (int64_t)b * s_blk] = w1;
  }
}

// SwiGLU backward of one row per wave from G = dout_t W_down[e] (fp32), as
// in the bf16 path, that also encodes the bf16-rounded dH in 1 x 128 blocks
// (fp32 scales) or, MX, 1 x 32 blocks (a word of four E8M0 codes per 128
// columns), the words stored run-major ([I/64][R]): the A operand of the
// gate/up dgrad.  Lane l handles the 8-column
// chunks l, l + 64, ... of the gate and of the up half; a 16-lane group
// covers 128 columns.  Requires I % 128 == 0.
template <bool MX>
__global__ __launch_bounds__(256) void swiglu_bwd_fp8_kernel(
    const f32x4_t* __restrict__ G, const u32x4_t* __restrict__ H, const float* __restrict__ topk_w,
    const int32_t* __restrict__ src_of, int R, int chunks, u32x4_t* __restrict__ dH,
    float* __restrict__ dw, uint8_t* __restrict__ dhq, uint32_t* __restrict__ dhs) {
  // dH scale words run-major: word (row r, 128-column block j) at dhs[j * R + r]
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int lane = threadIdx.x & 63;
  const float wr = topk_w[src_of[r]];
  const f32x4_t* Gr = G + (int64_t)r * 2 * chunks;  // 8 columns = two float4
  const u32x4_t* Hg = H + (int64_t)r * 2 * chunks;
  u32x4_t* Dr = dH + (int64_t)r * 2 * chunks;
  uint8_t* Qr = dhq + (int64_t)r * 2 * chunks * 8;
  uint32_t* Sr = dhs + r;
  float part = 0.0f;
  for (int c0 = 0; c0 < chunks; c0 += kWave) {  // uniform trip count
    const int c = c0 + lane;
    const bool ok = c < chunks;  // whole 16-lane groups share ok (chunks % 16 == 0)
    float gv[8], g[8], u[8], dg[8], du[8];
    u32x4_t zero = {0, 0, 0, 0};
    const f32x4_t fz = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t g0 = ok ? Gr[2 * c] : fz, g1 = ok ? Gr[2 * c + 1] : fz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gv[i] = g0[i];
      gv[4 + i] = g1[i];
    }
    unpack8(ok ? Hg[c] : zero, g);
    unpack8(ok ? Hg[chunks + c] : zero, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = sigmoidf_(g[i]);
      part += gv[i] * (g[i] * sg * u[i]);
      const float dA = wr * gv[i];
      dg[i] = dA * u[i] * sg * (1.0f + g[i] * (1.0f - sg));
      du[i] = dA * g[i] * sg;
    }
    // bf16 rounding first: the codes encode the stored dH
    u32x4_t pg, pu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pg[i] = pack_bf16x2(dg[2 * i], dg[2 * i + 1]);
      pu[i] = pack_bf16x2(du[2 * i], du[2 * i + 1]);
    }
    unpack8(pg, dg);
    unpack8(pu, du);
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ag = fmaxf(ag, fabsf(dg[i]));
      au = fmaxf(au, fabsf(du[i]));
    }
    u32x2_t qg, qu;
    uint32_t wg, wu;
    if constexpr (MX) {  // four lanes per 32-column block
#pragma unroll
      for (int off = 2; off >= 1; off >>= 1) {
        ag = fmaxf(ag, __shfl_xor(ag, off, kWave));
        au = fmaxf(au, __shfl_xor(au, off, kWave));
      }
      const MxScale sgate = mx_scale(ag), sup = mx_scale(au);
      qg = quant8_mx(dg, sgate.inv);
      qu = quant8_mx(du, sup.inv);
      wg = gather4_codes(sgate.code, lane & ~15, 4);
      wu = gather4_codes(sup.code, lane & ~15, 4);
    } else {
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        ag = fmaxf(ag, __shfl_xor(ag, off, kWave));
        au = fmaxf(au, __shfl_xor(au, off, kWave));
      }
      const float sgate = block_scale(ag), sup = block_scale(au);
      qg = quant8(dg, sgate);
      qu = quant8(du, sup);
      wg = __float_as_uint(sgate);
      wu = __float_as_uint(sup);
    }
    if (ok) {
      Dr[c] = pg;
      Dr[chunks + c] = pu;
      *(u32x2_t*)(Qr + c * 8) = qg;
      *(u32x2_t*)(Qr + (chunks + c) * 8) = qu;
      if ((lane & 15) == 0) {
        Sr[(int64_t)(c / 16) * R] = wg;
        Sr[(int64_t)((chunks + c) / 16) * R] = wu;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
  if (lane == 0) dw[r] = part;
}

}  // namespace

hipError_t launch_swiglu_bwd_fp8(const LaunchCtx& c, const float* G, const void* H,
                                 const float* topk_w, const int32_t* src_of, int R, int I, void* dH,
                                 float* dw, uint8_t* dhq, void* dhs, bool mx) {
  if (mx)
    MOE_LAUNCH(c, "swiglu_bwd", swiglu_bwd_fp8_kernel<true>, dim3((R + 3) / 4), dim3(256), 0,
               (const f32x4_t*)G, (const u32x4_t*)H, topk_w, src_of, R, I / 8, (u32x4_t*)dH, dw, dhq,
               (uint32_t*)dhs);
  else
    MOE_LAUNCH(c, "swiglu_bwd", swiglu_bwd_fp8_kernel<false>, dim3((R + 3) / 4), dim3(256), 0,
               (const f32x4_t*)G, (const u32x4_t*)H, topk_w, src_of, R, I / 8, (u32x4_t*)dH, dw, dhq,
               (uint32_t*)dhs);
  return hipSuccess;
}

hipError_t launch_quant_rows(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                             int64_t rows, int C, uint8_t* q, void* s, bool mx, bool run_major,
                             const int32_t* row_of, int k) {
  const int64_t nb = rows * (C / 128);
  if (nb == 0) return hipSuccess;
  const int64_t srows = row_of ? rows * k : rows;  // rows of the scale words
  const int64_t s_row = (run_major || row_of) ? 1 : C / 128, s_blk = (run_major || row_of) ? srows : 1;
  if (mx)
    MOE_LAUNCH(c, name, quant_rows_kernel<true>, dim3((unsigned)cdiv(nb, 16)), dim3(256), 0,
               (const bf16_t*)src, ld, rows, C, q, s, s_row, s_blk, row_of, k);
  else
    MOE_LAUNCH(c, name, quant_rows_kernel<false>, dim3((unsigned)cdiv(nb, 16)), dim3(256), 0,
               (const bf16_t*)src, ld, rows, C, q, s, s_row, s_blk, row_of, k);
  return hipSuccess;
}

hipError_t launch_quant_weight(const LaunchCtx& c, const char* name, const void* W, int E, int N,
                               int K, uint8_t* q, float* s, uint8_t* qt, float* st) {
  MOE_LAUNCH(c, name, quant_weight_kernel, dim3(K / 128, N / 128, E), dim3(256), 0,
             (const bf16_t*)W, N, K, q, s, qt, st);
  return hipSuccess;
}

hipError_t launch_quant_weight_mx(const LaunchCtx& c, const char* name, const void* W, int E, int N,
                                  int K, uint8_t* q, uint8_t* s, uint8_t* qt, uint8_t* st, bool run_major) {
  MOE_LAUNCH(c, name, quant_weight_mx_kernel, dim3(K / 128, N / 128, E), dim3(256), 0,
             (const bf16_t*)W, N, K, q, s, qt, st, (int)run_major);
  return hipSuccess;
}

hipError_t launch_quant_tok(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                            const int32_t* src_of, int kdiv, int C, const int32_t* offsets,
                            const int32_t* blk_off, int E, int nblk_max, uint8_t* q, void* s,
                            bool mx, bool run_major) {
  const int64_t s_row = run_major ? 1 : nblk_max, s_blk = run_major ? C : 1;
  if (mx)
    MOE_LAUNCH(c, name, quant_tok_kernel<true>, dim3(nblk_max, C / kTokCols), dim3(256), 0,
               (const bf16_t*)src, ld, src_of, kdiv, offsets, blk_off, E, q, (int64_t)nblk_max * 128,
               (uint32_t*)s, s_row, s_blk);
  else
    MOE_LAUNCH(c, name, quant_tok_kernel<false>, dim3(nblk_max, C / kTokCols), dim3(256), 0,
               (const bf16_t*)src, ld, src_of, kdiv, offsets, blk_off, E, q, (int64_t)nblk_max * 128,
               (uint32_t*)s, s_row, s_blk);
  return hipSuccess;
}

}  // namespace moe
