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

using tile::u32x2_t;
using tile::u32x4_t;

constexpr float kE4M3Max = 448.0f;

// Scale of a block with largest magnitude amax (correctly rounded division).
__device__ __forceinline__ float block_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
}

// Blockwise quotients f[i] <- RN(f[i] / s), i < N, for the e4m3 encoding
// (whose codes are the e4m3 rounding of the rounded quotient).  With
// rs = RN(1 / s), q = RN(f rs) lies within an ulp of the quotient, and one
// FMA correction, RN(q + RN(f - q s) rs), gives the rounded quotient
// exactly (Markstein's theorem on FMA-based division) as long as the
// residual f - q s does not underflow: here |f| >= 2^-100, and rs finite.
// Zero keeps its sign through q.  A wave with any other value in any lane
// (a nonzero magnitude below 2^-100, or a block whose scale lies below
// 2^-128, where rs overflows) divides all of its values instead: one
// wave-uniform branch, which ordinary data never enters.
//
// quot_run divides f[0, N) by s, and quot_run2 two runs by their own
// scales; then `use` consumes the quotients, inside each branch.  Uniform,
// and with nothing merging after it, the branch costs no registers: a
// divergent one would keep every original value live through the division
// side for the other lanes (50 more registers in the weight quantiser).
__device__ __forceinline__ bool quot_slow(float v) { return v != 0.0f && fabsf(v) < 0x1p-100f; }
__device__ __forceinline__ bool quot_rs_ok(float rs) { return rs <= 0x1.fffffep+127f; }

template <int N>
__device__ __forceinline__ void quot_divide(float* f, float s) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    f[i] = __fdiv_rn(f[i], s);
    __builtin_amdgcn_sched_barrier(0);  // one at a time: interleaved, they would set the register budget
  }
}

template <int N>
__device__ __forceinline__ void quot_fma(float* f, float s, float rs) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float q = f[i] * rs;
    f[i] = f[i] == 0.0f ? q : fmaf(fmaf(-q, s, f[i]), rs, q);
  }
}

template <int N, class F>
__device__ __forceinline__ void quot_run(float* f, float s, float rs, F&& use) {
  bool slow = !quot_rs_ok(rs);
#pragma unroll
  for (int i = 0; i < N; ++i) slow |= quot_slow(f[i]);
  if (__builtin_amdgcn_ballot_w64(slow)) quot_divide<N>(f, s);
  else quot_fma<N>(f, s, rs);
  use();
}

template <int N, class F>
__device__ __forceinline__ void quot_run2(float* f0, float s0, float r0, float* f1, float s1, float r1, F&& use) {
  bool slow = !quot_rs_ok(r0) || !quot_rs_ok(r1);
#pragma unroll
  for (int i = 0; i < N; ++i) slow |= quot_slow(f0[i]) || quot_slow(f1[i]);
  if (__builtin_amdgcn_ballot_w64(slow)) {
    quot_divide<N>(f0, s0);
    quot_divide<N>(f1, s1);
  } else {
    quot_fma<N>(f0, s0, r0);
    quot_fma<N>(f1, s1, r1);
  }
  use();
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

// Lane exchanges within a row of 16 lanes by DPP (no LDS trip): quad
// permutations 0xB1 (the lane xor 1) and 0x4E (xor 2), and the half-row
// mirror (lane i of each 8 takes lane 7 - i).
constexpr int kHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Reduction over the four lanes 4m .. 4m + 3 of a quad: combine with the
// lane xor 1, then with the lane xor 2.
template <class Op>
__device__ __forceinline__ float quad_reduce(float v, Op op) {
  v = op(v, dpp_f32<0xB1>(v));
  return op(v, dpp_f32<0x4E>(v));
}
__device__ __forceinline__ float quad_max(float v) {
  return quad_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// Eight values divided by s, as eight e4m3 codes.
__device__ __forceinline__ u32x2_t quant8(const float (&f)[8], float s) {
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = f[i];
  u32x2_t q;
  quot_run<8>(g, s, __fdiv_rn(1.0f, s), [&] {
    q[0] = e4m3x4(g[0], g[1], g[2], g[3]);
    q[1] = e4m3x4(g[4], g[5], g[6], g[7]);
  });
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
  // 128 rows x 128 bytes: chunk c = 16 bytes (4 words) of row c / 8.  The
  // stores are non-temporal: a weight's codes (as large as half the weight)
  // are read by a GEMM only after the whole weight is encoded, far beyond
  // what L2 keeps (weight quantisers 1-4% faster than with cached stores).
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = p * 256 + threadIdx.x;
    const int row = c >> 3, w = (c & 7) * 4;
    const uint32_t* src = tile + row * kWS + w;
    __builtin_nontemporal_store(u32x4_t{src[0], src[1], src[2], src[3]}, (u32x4_t*)(dst + (int64_t)row * ld + w * 4));
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
    // non-temporal (cache policy nt): the weight is read once
    __builtin_amdgcn_global_load_lds(Wb + (int64_t)row * K + c * 8, (tile::lds_void_t*)(stage + q * 1024), 16, 0, 2);
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
  quot_run<64>(&f[0][0], sc, rsc, [&] {
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
  });
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
// src_of[r] / kdiv (token rows of x or dout) or r.  A work-group handles
// cpw chunks of 64 columns, one after the other: q[c][128 b + i] = code (0
// past the segment) and the scale word of (column c, run b) at
// s[c * s_row + b * s_blk]: the run's fp32 scale or, MX, the E8M0 codes of
// its four 32-row blocks.  Run-major words (s_row = 1, s_blk = columns) put
// the words of one run for consecutive columns side by side, as one K step
// of the weight-gradient GEMMs reads them.
//
// The run's expert, first row and source rows take a chain of dependent
// loads (the search over blk_off, offsets, src_of); walking several column
// chunks per work-group pays that chain once for all of them, and each
// chunk's loads leave while the previous chunk is encoded.
// ---------------------------------------------------------------------------
constexpr int kTokCols = 64;

// One 128-row x 64-column chunk of quant_tok_kernel, staged in tile.
template <bool MX>
__device__ __forceinline__ void quant_tok_chunk(const uint8_t* tile, int t, int c0, int b,
                                                uint8_t* __restrict__ q, int64_t ldq,
                                                uint32_t* __restrict__ s, int64_t s_row, int64_t s_blk) {
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
    a0 = fmaxf(a0, dpp_f32<0xB1>(a0));
    a1 = fmaxf(a1, dpp_f32<0xB1>(a1));
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
    a0 = quad_max(a0);  // then the other quad of the eight lanes rg
    a1 = quad_max(a1);
    a0 = fmaxf(a0, dpp_f32<kHalfMirror>(a0));
    a1 = fmaxf(a1, dpp_f32<kHalfMirror>(a1));
    const float s0 = block_scale(a0), s1 = block_scale(a1);
    const float r0 = __fdiv_rn(1.0f, s0), r1 = __fdiv_rn(1.0f, s1);
    quot_run2<16>(f0, s0, r0, f1, s1, r1, [&] {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        q0[w] = e4m3x4(f0[4 * w], f0[4 * w + 1], f0[4 * w + 2], f0[4 * w + 3]);
        q1[w] = e4m3x4(f1[4 * w], f1[4 * w + 1], f1[4 * w + 2], f1[4 * w + 3]);
      }
    });
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

template <bool MX>
__global__ __launch_bounds__(256) void quant_tok_kernel(const bf16_t* __restrict__ src, int64_t ld,
                                                       const int32_t* __restrict__ src_of, int kdiv,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ blk_off, int E,
                                                       uint8_t* __restrict__ q, int64_t ldq,
                                                       uint32_t* __restrict__ s, int64_t s_row, int64_t s_blk,
                                                       int cpw) {
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
  const int t = threadIdx.x;
  // this thread's four source rows (i = t/8 + 32 p), 16 bytes of each per chunk
  const bf16_t* rp[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = (t >> 3) + 32 * p;
    rp[p] = nullptr;
    if (i < n) {
      const int64_t sr = src_of ? (int64_t)(src_of[r0 + i] / kdiv) : (int64_t)(r0 + i);
      rp[p] = src + sr * ld + (t & 7) * 8;
    }
  }
  u32x4_t v[4];
  auto load = [&](int c0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) v[p] = rp[p] ? *(const u32x4_t*)(rp[p] + c0) : u32x4_t{0, 0, 0, 0};
  };
  int c0 = blockIdx.y * cpw * kTokCols;
  load(c0);
  for (int j = 0; j < cpw; ++j, c0 += kTokCols) {
    if (j) __syncthreads();  // the previous chunk's tile reads are done
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      u32x2_t* dst = (u32x2_t*)(tile + ((t >> 3) + 32 * p) * 136 + (t & 7) * 16);
      dst[0] = u32x2_t{v[p][0], v[p][1]};
      dst[1] = u32x2_t{v[p][2], v[p][3]};
    }
    if (j + 1 < cpw) load(c0 + kTokCols);
    __syncthreads();
    quant_tok_chunk<MX>(tile, t, c0, b, q, ldq, s, s_row, s_blk);
  }
}

// SwiGLU backward with both fp8 encodings of dH, for the blockwise and MX
// backwards: one work-group per (128-row run of an expert's segment, 128
// columns of I), as quant_tok_kernel's runs.  From G = dout_t W_down[e]
// (fp32) and the stored H it forms dH (bf16-rounded, as the bf16 path
// stores it; clamp lim as there), then encodes it twice without writing it:
// rows in 1 x 128 blocks (blockwise fp32 scales) or 1 x 32 (MX), the gate/up
// dgrad's operand (codes dhq [R, 2I], words run-major dhs [2I/128][R]); and
// columns in the run's 128-row blocks (or 32-row, MX), transposed, the
// gate/up wgrad's operand (q [2I][128 nblk], words as quant_tok_kernel's).
// It also writes <G_r, a_r> over its 128 columns to dw[r * (I/128) + chunk].
// Thread t: row t / 4 of the run, the four 8-column pieces 8 (t % 4) + 32 j
// of the chunk (gate and up).  The bf16 dH goes through LDS as four
// 128 x 64 tiles (gate 0-63, gate 64-127, up 0-63, up 64-127) for the
// column encoding.
template <bool MX>
__global__ __launch_bounds__(512) void swiglu_bwd_tok_kernel(
    const float* __restrict__ G, const bf16_t* __restrict__ H, const float* __restrict__ topk_w,
    const int32_t* __restrict__ src_of, int R, int I, float lim, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ blk_off, int E, float* __restrict__ dw, uint8_t* __restrict__ dhq,
    uint32_t* __restrict__ dhs, uint8_t* __restrict__ q, int64_t ldq, uint32_t* __restrict__ s,
    int64_t s_row, int64_t s_blk) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][128 * 136];
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
  const int chunk = blockIdx.y, c0 = chunk * 128;
  const int t = threadIdx.x, i = t >> 2, qd = t & 3;
  const bool ok = i < n;
  const int64_t r = r0 + (ok ? i : 0);
  const float wr = ok ? topk_w[src_of[r]] : 0.0f;
  // chunk j (0..3) of this thread: columns c0 + 8 qd + 32 j .. +7, so the
  // four threads of a row read 32 (gate/up: 16) contiguous bytes each
  const float* Gr = G + r * I + c0 + 8 * qd;
  const bf16_t* Hg = H + r * 2 * I + c0 + 8 * qd;
  const bf16_t* Hu = Hg + I;
  f32x4_t gr[8];
  u32x4_t hg[4], hu[4];
  const f32x4_t fz = {0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4_t uz = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    gr[2 * j] = ok ? *(const f32x4_t*)(Gr + 32 * j) : fz;
    gr[2 * j + 1] = ok ? *(const f32x4_t*)(Gr + 32 * j + 4) : fz;
    hg[j] = ok ? *(const u32x4_t*)(Hg + 32 * j) : uz;
    hu[j] = ok ? *(const u32x4_t*)(Hu + 32 * j) : uz;
  }
  u32x4_t pg[4], pu[4];  // bf16 dH of chunk j, packed pairs
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float g[8], u[8];
    unpack8(hg[j], g);
    unpack8(hu[j], u);
#pragma unroll
    for (int m = 0; m < 8; m += 2) {
      float dg[2], du[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const float gv = gr[2 * j + ((m + x) >> 2)][(m + x) & 3];
        const float gc = clamp_gate(g[m + x], lim), uc = clamp_up(u[m + x], lim);
        const float sg = sigmoidf_(gc);
        part += gv * (gc * sg * uc);
        const float dA = wr * gv;
        dg[x] = g[m + x] <= lim ? dA * uc * sg * (1.0f + gc * (1.0f - sg)) : 0.0f;
        du[x] = fabsf(u[m + x]) <= lim ? dA * gc * sg : 0.0f;
      }
      pg[j][m >> 1] = pack_bf16x2(dg[0], dg[1]);
      pu[j][m >> 1] = pack_bf16x2(du[0], du[1]);
    }
  }
  // the bf16 dH into the column-encoding tiles (column c of the chunk: tile
  // c / 64, byte 2 (c % 64) of a 136-byte row)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int off = i * 136 + 16 * qd + 64 * (j & 1);
    *(u32x4_t*)(tiles[j >> 1] + off) = pg[j];
    *(u32x4_t*)(tiles[2 + (j >> 1)] + off) = pu[j];
  }
  // dw partial over the chunk's 128 columns (four threads of the row)
  part = quad_reduce(part, [](float a, float b) { return a + b; });
  if (ok && qd == 0) dw[r * (I / 128) + chunk] = part;
  // row encodings of the gate (half 0) and up (half 1) columns: a 1 x 128
  // block spans the four threads of the row; MX block j is their chunks j
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float f[4][8], am[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unpack8(half ? pu[j] : pg[j], f[j]);
      am[j] = 0.0f;
#pragma unroll
      for (int x = 0; x < 8; ++x) am[j] = fmaxf(am[j], fabsf(f[j][x]));
    }
    u32x2_t code[4];
    uint32_t word;
    if constexpr (MX) {
      word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const MxScale sc = mx_scale(quad_max(am[j]));
        code[j] = quant8_mx(f[j], sc.inv);
        word |= sc.code << (8 * j);
      }
    } else {
      const float sc = block_scale(quad_max(fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3]))));
      quot_run<32>(&f[0][0], sc, __fdiv_rn(1.0f, sc), [&] {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          code[j][0] = e4m3x4(f[j][0], f[j][1], f[j][2], f[j][3]);
          code[j][1] = e4m3x4(f[j][4], f[j][5], f[j][6], f[j][7]);
        }
      });
      word = __float_as_uint(sc);
    }
    if (ok) {
      const int col = half * I + c0;
      uint8_t* dq = dhq + r * 2 * I + col + 8 * qd;
#pragma unroll
      for (int j = 0; j < 4; ++j) *(u32x2_t*)(dq + 32 * j) = code[j];
      if (qd == 0) dhs[(int64_t)(col >> 7) * R + r] = word;
    }
  }
  __syncthreads();
  // column encodings: threads 0-255 the gate tiles, 256-511 the up tiles
  const int grp = t >> 8, tt = t & 255;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    quant_tok_chunk<MX>(tiles[2 * grp + k], tt, grp * I + c0 + 64 * k, b, q, ldq, s, s_row, s_blk);
}

}  // namespace

hipError_t launch_swiglu_bwd_tok(const LaunchCtx& c, const float* G, const void* H, const float* topk_w,
                                 const int32_t* src_of, int R, int I, float lim, const int32_t* offsets,
                                 const int32_t* blk_off, int E, int nblk_max, float* dw, uint8_t* dhq,
                                 void* dhs, uint8_t* q, void* s, bool mx) {
  // token-block words run-major (s_row = 1, s_blk = 2I), as quant_tok's
  const int64_t s_row = 1, s_blk = 2 * (int64_t)I, ldq = (int64_t)nblk_max * 128;
  const dim3 grid(nblk_max, I / 128);
  if (mx)
    MOE_LAUNCH(c, "swiglu_bwd", swiglu_bwd_tok_kernel<true>, grid, dim3(512), 0, G, (const bf16_t*)H, topk_w,
               src_of, R, I, lim, offsets, blk_off, E, dw, dhq, (uint32_t*)dhs, q, ldq, (uint32_t*)s, s_row,
               s_blk);
  else
    MOE_LAUNCH(c, "swiglu_bwd", swiglu_bwd_tok_kernel<false>, grid, dim3(512), 0, G, (const bf16_t*)H, topk_w,
               src_of, R, I, lim, offsets, blk_off, E, dw, dhq, (uint32_t*)dhs, q, ldq, (uint32_t*)s, s_row,
               s_blk);
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
  // column chunks per work-group: up to 8, dividing C / 64, while the grid
  // keeps at least 2048 work-groups
  const int chunks = C / kTokCols;
  int cpw = 8;
  while (cpw > 1 && (chunks % cpw || (int64_t)nblk_max * (chunks / cpw) < 2048)) cpw >>= 1;
  if (mx)
    MOE_LAUNCH(c, name, quant_tok_kernel<true>, dim3(nblk_max, C / kTokCols / cpw), dim3(256), 0,
               (const bf16_t*)src, ld, src_of, kdiv, offsets, blk_off, E, q, (int64_t)nblk_max * 128,
               (uint32_t*)s, s_row, s_blk, cpw);
  else
    MOE_LAUNCH(c, name, quant_tok_kernel<false>, dim3(nblk_max, C / kTokCols / cpw), dim3(256), 0,
               (const bf16_t*)src, ld, src_of, kdiv, offsets, blk_off, E, q, (int64_t)nblk_max * 128,
               (uint32_t*)s, s_row, s_blk, cpw);
  return hipSuccess;
}

}  // namespace moe
