// Grouped GEMMs of the expert MLPs on block-scaled fp8 operands (OCP e4m3)
// on gfx950 MFMA with fp32 accumulation, in two scale formats ("Prime
// Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster", section
// "Precision and hardware support": blockwise FP8, and MXFP8 with smaller
// scaling groups).
//
// Every operand arrives quantised and contiguous along K (see
// quant_fp8.hip), K is a multiple of 128, and each output tile takes one
// v_mfma_scale_f32_16x16x128_f8f6f4 per K step of 128.
//   blockwise: one K step is exactly one fp32 scale block.  The MFMA runs
//     with unit block exponents into a fresh partial sum P, which is promoted
//     into the fp32 accumulator with the product of the two operands'
//     scales: acc += P * (s_row * s_col).
//   MX: every lane hands the MFMA the E8M0 codes of its row's 32-value block
//     (lane l: row l % 16, block l / 16 of the step), so the instruction
//     applies the scales itself and accumulates straight into acc.
//
// Tile engine: 256 (token rows) x 256 (features) per work-group, eight waves
// of 128 x 64, 128 bytes of K per stage for both operands (the same 64 KB
// per stage as the bf16 engine, for twice the MFMA work).  Operands and one
// 32-bit scale word per row and K step (an fp32 scale, or four E8M0 codes)
// move global -> LDS with direct loads into a two-stage ring.  The scale
// words are stored run-major wherever a step's words would otherwise sit one
// per cache line (expert-sorted activations, x's and dout's words written
// per expert-sorted row, MX weights, token runs), so a step's 256 words are
// one contiguous kilobyte.  The MFMA's A operand is the feature side and its
// B operand the token side, so a lane's four results share one token row:
// the blockwise promotion costs one multiply-add per result, and it runs a
// sub-step behind the MFMAs that produced the partial.
#include <type_traits>

#include "common.h"
#include "tile.h"

namespace moe {
namespace {
using namespace tile;

constexpr int KB = 128;                // K per stage (bytes = e4m3 elements)
constexpr int NWAVE = 8;
constexpr int NTHR = NWAVE * 64;
constexpr int WM = 2, WN = 4;          // wave grid: token halves x feature quarters
constexpr int TBM = 256, TBN = 256;    // tokens x features per work-group
constexpr int TM = TBM / WM / 16;      // 16-row MFMA tiles per wave along tokens (8)
constexpr int TN = TBN / WN / 16;      // along features (4)
constexpr int OPB = TBM * KB;          // bytes of one operand per stage
constexpr int SCB = 256 * 4;           // bytes of one side's scales per stage
constexpr int STB = 2 * OPB + 2 * SCB; // stage: token op | feature op | token scales | feature scales
static_assert(TBM == kRowTile, "tile table is built for 256-row tiles");

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// Where the feature side's scales come from.
enum ScaleMode {
  SC_WEIGHT = 0,  // blockwise, one scale per 128 feature rows (a weight)
  SC_ROW = 1,     // blockwise, one scale per feature row (token-blocked operand)
  SC_MX = 2,      // MX: E8M0 codes per row and 32-value block, both sides
};

// LDS operand layout: [row][128 bytes], 16-byte chunk c of row r stored at
// position c ^ swz8(r).  The swizzle depends on row bits 1..3 only, so the 16
// rows of an MFMA fragment (16-aligned) read at one chunk cover all 16 slots
// of a 256-byte bank window, and a lane's address for any 16-aligned row base
// is its own offset plus a constant.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// ---------------------------------------------------------------------------
// One operand: 64 NI rows x 128 bytes per stage (NI = 4: 256 rows).
// Instruction q covers rows 8q..8q+7 (1 KB); wave w issues q = w + 8i, i < NI.
// ---------------------------------------------------------------------------
struct FragOff;

template <int NI = 4>
struct Op8 {
  static constexpr int N = NI;
  const uint8_t* ptr[NI];  // this lane's 16-byte chunk at the current stage

  __device__ static int koff(int i) {
    const int lane = threadIdx.x & 63;
    const int row = 8 * ((threadIdx.x >> 6) + NWAVE * i) + (lane >> 3);
    return ((lane & 7) ^ swz8(row)) << 4;
  }
  // rowp(row) -> first byte of the row's K range
  template <class F>
  __device__ void init(F rowp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] = rowp(8 * (w + NWAVE * i) + (lane >> 3)) + koff(i);
  }
  template <int I0, int I1>
  __device__ void issue(lds_t* s) const {
    const int w = wave_id();
#pragma unroll
    for (int i = I0; i < (I1 < NI ? I1 : NI); ++i) dma16(ptr[i], s + (w + NWAVE * i) * 1024);
  }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] += KB;
  }
  __device__ static i32x8_t frag(const lds_t* fb, int n0, const FragOff& fo);  // after frag8
};

// MFMA operand of 16 rows in the instruction's K order: lane l holds row
// l % 16 of the fragment and, with g = l / 16, K bytes 16 g .. 16 g + 15 in
// its first four registers and 64 + 16 g .. +15 in the last four (chunks g
// and g + 4 of the stage).  The instruction's 32-value scale block b is then
// K bytes 32 b .. 32 b + 31, as the MX operands are encoded.
struct FragOff {
  int lo, hi;  // byte offsets of this lane's two chunks from the fragment's first row
  __device__ FragOff() {
    const int lane = threadIdx.x & 63, r = lane & 15, c = lane >> 4;
    lo = r * KB + ((c ^ swz8(r)) << 4);
    hi = r * KB + (((c + 4) ^ swz8(r)) << 4);
  }
};
__device__ __forceinline__ i32x8_t frag8(const lds_t* s, const FragOff& o) {
  const u32x4_t lo = *(const __attribute__((address_space(3))) u32x4_t*)(s + o.lo);
  const u32x4_t hi = *(const __attribute__((address_space(3))) u32x4_t*)(s + o.hi);
  const i32x8_t r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return r;
}

// Feature fragment (16 features from n0, one K step) of a stage whose
// feature operand is stored [row][128 K bytes].
template <int NI>
__device__ __forceinline__ i32x8_t Op8<NI>::frag(const lds_t* fb, int n0, const FragOff& fo) {
  return frag8(fb + n0 * KB, fo);
}

// ---------------------------------------------------------------------------
// Feature operand whose memory rows run along the features: element (n, k)
// at base[k * ld + n] (a blockwise weight read in its forward layout by a
// data gradient, where the contraction runs over the weight's rows).  A stage
// is 128 k-rows of the tile's 256 features, 256 bytes each; row k's 16-byte
// chunk c sits at chunk c ^ kn_swz(k).  Instruction q covers k-rows 4q ..
// 4q+3 (1 KB); wave w issues q = w + 8i, i < 4.  Features at or past N read
// the row's first chunk (computed, never stored).
//
// Fragments come from ds_read_b64_tr_b8.  Within each 16-lane group, lane i
// < 8 receives byte i of the 8 bytes that lanes 0, 2, .., 14 address, lane
// 8 + i byte i of those of lanes 1, 3, .., 15 (probed).  So with lane s
// addressing k-row k0 + s / 2 at feature n0 + 8 (s % 2), lane i gets K bytes
// k0 .. k0 + 7 of feature n0 + i: the MFMA's own layout (lane l: feature l %
// 16, K bytes 16 g .. 16 g + 15 and 64 + 16 g .. + 15, g = l / 16) takes
// four such reads.  The swizzle folds row bit 4 into bit 3 so that the 32
// k-rows one read covers spread over all chunk positions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kn_swz(int k) { return (k & 15) ^ (((k >> 4) & 1) << 3); }

struct Op8KN {
  static constexpr int N = 4;
  const uint8_t* ptr[N];  // this lane's 16-byte chunk at the current stage
  int64_t step;           // bytes per K step (128 rows)

  // base: element (feature of the tile's first column, k = 0); nvalid:
  // features of the tile inside N
  __device__ void init(const uint8_t* base, int64_t ld, int nvalid) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    step = (int64_t)KB * ld;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = 4 * (w + NWAVE * i) + (lane >> 4);
      int c = (lane & 15) ^ kn_swz(row);
      if (c * 16 >= nvalid) c = 0;
      ptr[i] = base + (int64_t)row * ld + c * 16;
    }
  }
  template <int I0, int I1>
  __device__ void issue(lds_t* s) const {
    const int w = wave_id();
#pragma unroll
    for (int i = I0; i < (I1 < N ? I1 : N); ++i) dma16(ptr[i], s + (w + NWAVE * i) * 1024);
  }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < N; ++i) ptr[i] += step;
  }
  __device__ static i32x8_t frag(const lds_t* fb, int n0, const FragOff&) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63, sl = lane & 15, g = lane >> 4;
    const int cb = n0 >> 4, byte = 8 * (sl & 1);
    v2i r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 16 * g + 8 * (q & 1) + 64 * (q >> 1) + (sl >> 1);
      r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(fb + k * (TBN) + ((cb ^ kn_swz(k)) << 4) + byte));
    }
    const i32x8_t f = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    return f;
  }
};
static_assert(TBN == 256 && KB * TBN == OPB, "Op8KN stage: 128 k-rows of 256 features");

__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) / WN; }
__device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) % WN; }

// Scales: waves 0-3 load the token rows' scale words (rows 64w .. 64w+63),
// waves 4-7 the feature rows' (rows 64(w-4) ..); sp is the lane's source at
// the current stage, advanced by sstep words per K step (1 for row-major
// words, the row count for run-major ones).

// Part I of a stage's loads: token-operand instruction I / 2 (even I) or
// feature-operand instruction I / 2 (odd I); part 0 adds the scales.
template <int I, class OT, class OF>
__device__ __forceinline__ void issue_step(const OT& ot, const OF& of, const uint32_t* sp, lds_t* dst) {
  constexpr int q = I / 2;
  if constexpr (I % 2 == 0) ot.template issue<q, q + 1>(dst);
  else of.template issue<q, q + 1>(dst + OPB);
  if constexpr (I == 0) dma4(sp, dst + 2 * OPB + 256 * wave_id());
}

template <class OT, class OF>
__device__ __forceinline__ void issue_stage(const OT& ot, const OF& of, const uint32_t* sp, lds_t* dst) {
  issue_step<0>(ot, of, sp, dst); issue_step<1>(ot, of, sp, dst); issue_step<2>(ot, of, sp, dst);
  issue_step<3>(ot, of, sp, dst); issue_step<4>(ot, of, sp, dst); issue_step<5>(ot, of, sp, dst);
  issue_step<6>(ot, of, sp, dst); issue_step<7>(ot, of, sp, dst);
}

// ---------------------------------------------------------------------------
// Main loop over nkb K steps.  TMX: 16-row MFMA tiles per wave along tokens
// (8 for a 256-row tile; 4 / 2 for a segment tail of at most 128 / 64 rows,
// whose token operand is loaded for 128 / 64 rows only).  SC_ROW: the
// feature side has a scale per row (token-blocked operands) rather than per
// 128 rows (weights), so each of a lane's four results takes its own
// feature scale.
// acc[i][j][r]: token wave_m*16*TMX + 16 i + lane % 16, feature
// wave_n*64 + 16 j + 4 (lane / 16) + r.
// ---------------------------------------------------------------------------
// acc += P s_token s_feature for one sub-tile row's TN partials.  With
// weight scales (SC_WEIGHT) a wave's 64 features lie in one 128-row weight
// block, or, in the gate/up GEMM, in one 32-row block of gate rows (tiles 0,
// 1) and one of up rows (tiles 2, 3): tiles 0 and 1 share a scale, as do 2
// and 3, so two products serve all four (the same floats, so the same
// results as one product per tile, with a quarter of the multiplies).
static_assert(TN == 4, "feature tiles per wave");
template <int SC>
__device__ __forceinline__ void promote(f32x4_t (&acc)[TN], const f32x4_t (&P)[TN], float sa,
                                        const f32x4_t (&sb)[TN]) {
  if constexpr (SC == SC_ROW) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(P[j][r] * sb[j][r], sa, acc[j][r]);
  } else {
    const float s01 = sa * sb[0][0], s23 = sa * sb[2][0];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(P[j][r], j < 2 ? s01 : s23, acc[j][r]);
  }
}

// Blockwise sub-step I: its MFMAs write fresh partials P[I & 1]; the
// partials of sub-step I - 1, whose MFMAs issued a whole sub-step earlier,
// are promoted after them (so no FMA waits on the MFMA it follows), with
// that sub-step's token scale sap.  The last sub-step's partials are
// promoted by the caller.
template <int SC, int TMX, bool PRE, int I, class OT, class OF>
__device__ __forceinline__ void substep(const OT& ot, const OF& of, const uint32_t* sp, lds_t* dst,
                                        const i32x8_t (&f)[TN], const i32x8_t& t,
                                        const lds_f32_t* SAw, float& sa, float& sap, const f32x4_t (&sb)[TN],
                                        f32x4_t (&P)[2][TN], f32x4_t (&acc)[TMX][TN]) {
  if constexpr (PRE && I == 0) issue_stage(ot, of, sp, dst);  // the next stage leaves at the step's start
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < TN; ++j)
    P[I & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f[j], t, zero, 0, 0, 0, 127, 0, 127);
  if constexpr (I > 0) promote<SC>(acc[I - 1], P[(I - 1) & 1], sap, sb);
  if constexpr (I > 0 && SC == SC_WEIGHT) {
    // the promotion's FMAs interleaved with this sub-step's MFMAs (five VALU
    // after each), not queued behind all four: the blockwise row GEMMs ran
    // 2-5% faster; the token-blocked weight gradients (two VALU per value)
    // ran 0.5-1.7% slower that way and keep the compiler's order
#pragma unroll
    for (int q = 0; q < TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
  }
  sap = sa;
  if constexpr (I + 1 < TMX) sa = SAw[(I + 1) * 16];  // token scale of the next sub-step
  // keep the scheduler from hoisting later sub-steps' fragment reads and
  // MFMAs: each would hold its own registers live
  __builtin_amdgcn_sched_barrier(0);
}

// MX sub-step I: the MFMA applies the E8M0 codes (byte 0 of each scale
// operand) and accumulates in place.  st: this lane's token-row code of
// sub-tile I; sf[j]: its feature-row code of sub-tile j.
template <int TMX, bool PRE, int I, class OT, class OF>
__device__ __forceinline__ void substep_mx(const OT& ot, const OF& of, const uint32_t* sp, lds_t* dst,
                                           const i32x8_t (&f)[TN], const i32x8_t& t, const lds_u8_t* SAl,
                                           int& st, const int (&sf)[TN], f32x4_t (&acc)[TMX][TN]) {
  if constexpr (PRE && I == 0) issue_stage(ot, of, sp, dst);
#pragma unroll
  for (int j = 0; j < TN; ++j)
    acc[I][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f[j], t, acc[I][j], 0, 0, 0, sf[j], 0, st);
  if constexpr (I + 1 < TMX) st = SAl[(I + 1) * 16 * 4];  // token code of the next sub-step
  __builtin_amdgcn_sched_barrier(0);
}

// Sub-steps I .. TMX-1 of a K step: t[I & 1] holds sub-step I's token
// fragment, the other slot sub-step I + 1's; each slot is refilled for
// I + 2 once its sub-step has issued.
template <int SC, int TMX, bool PRE, int I, class OT, class OF>
__device__ __forceinline__ void substeps(const OT& ot, const OF& of, const uint32_t* sp, lds_t* dst,
                                         const i32x8_t (&f)[TN], i32x8_t (&t)[2], const lds_t* tb,
                                         const FragOff& fo, const lds_f32_t* SAw, float& sa, float& sap,
                                         const f32x4_t (&sb)[TN], f32x4_t (&P)[2][TN], const lds_u8_t* SAl,
                                         int& st, const int (&sf)[TN], f32x4_t (&acc)[TMX][TN]) {
  if constexpr (I < TMX) {
    if constexpr (SC == SC_MX) substep_mx<TMX, PRE, I>(ot, of, sp, dst, f, t[I & 1], SAl, st, sf, acc);
    else substep<SC, TMX, PRE, I>(ot, of, sp, dst, f, t[I & 1], SAw, sa, sap, sb, P, acc);
    if constexpr (I + 2 < TMX) t[I & 1] = frag8(tb + (I + 2) * 16 * KB, fo);
    substeps<SC, TMX, PRE, I + 1>(ot, of, sp, dst, f, t, tb, fo, SAw, sa, sap, sb, P, SAl, st, sf, acc);
  }
}

// One K step on the stage in `cur`; PRE: also load the next stage into `dst`
// (a branch-free body, so the sub-step boundaries hold).
template <int SC, int TMX, bool PRE, class OT, class OF>
__device__ __forceinline__ void kstep(OT& ot, OF& of, const uint32_t*& sp, int sstep, const lds_t* cur,
                                      lds_t* dst, const FragOff& fo, f32x4_t (&acc)[TMX][TN]) {
  const int wm = wave_m(), wn = wave_n();
  const int lane = threadIdx.x & 63;
  wait_vmcnt<0>();
  barrier_lds();
  const int trow = wm * TMX * 16;  // this wave's first token row
  // blockwise scales: fp32 [row]; MX: words [row] of 4 codes, this lane's
  // code at row lane % 16 of each sub-tile, block lane / 16
  const lds_f32_t* SAw = nullptr;
  const lds_u8_t* SAl = nullptr;
  float sa = 0.0f;
  int st = 0;
  f32x4_t sb[TN];
  int sf[TN];
  if constexpr (SC == SC_MX) {
    const int lo = (lane & 15) * 4 + (lane >> 4);
    SAl = (const lds_u8_t*)(cur + 2 * OPB) + trow * 4 + lo;
    const lds_u8_t* SBl = (const lds_u8_t*)(cur + 2 * OPB + SCB) + wn * 64 * 4 + lo;
    st = SAl[0];
#pragma unroll
    for (int j = 0; j < TN; ++j) sf[j] = SBl[j * 16 * 4];
  } else {
    const lds_f32_t* SB = (const lds_f32_t*)(cur + 2 * OPB + SCB);
    SAw = (const lds_f32_t*)(cur + 2 * OPB) + trow + (lane & 15);
    sa = SAw[0];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int fr = wn * 64 + j * 16 + 4 * (lane >> 4);
      if constexpr (SC == SC_ROW) sb[j] = *(const __attribute__((address_space(3))) f32x4_t*)(SB + fr);
      else if (j % 2 == 0) sb[j][0] = SB[fr];  // tiles 0, 2 (see promote)
    }
  }
  const lds_t* tb = cur + trow * KB;  // this wave's token rows
  i32x8_t f[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) f[j] = OF::frag(cur + OPB, wn * 64 + j * 16, fo);
  i32x8_t t[2];
  t[0] = frag8(tb, fo);
  if constexpr (TMX > 1) t[1] = frag8(tb + 16 * KB, fo);
  float sap = 0.0f;
  f32x4_t P[2][TN];
  substeps<SC, TMX, PRE, 0>(ot, of, sp, dst, f, t, tb, fo, SAw, sa, sap, sb, P, SAl, st, sf, acc);
  if constexpr (SC != SC_MX) promote<SC>(acc[TMX - 1], P[(TMX - 1) & 1], sap, sb);
  if constexpr (PRE) {
    ot.advance();
    of.advance();
    sp += sstep;
  }
}

template <int SC, int TMX, class OT, class OF>
__device__ __forceinline__ void mainloop8(OT& ot, OF& of, const uint32_t* sp, int sstep, int nkb, char* smem,
                                          f32x4_t (&acc)[TMX][TN]) {
#pragma unroll
  for (int i = 0; i < TMX; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (nkb <= 0) return;
  lds_t* const base = (lds_t*)smem;
  const FragOff fo;
  issue_stage(ot, of, sp, base);
  ot.advance();
  of.advance();
  sp += sstep;
  int slot = 0;
  for (int kb = 0; kb + 1 < nkb; ++kb) {
    kstep<SC, TMX, true>(ot, of, sp, sstep, base + slot * STB, base + (slot ^ 1) * STB, fo, acc);
    slot ^= 1;
  }
  kstep<SC, TMX, false>(ot, of, sp, sstep, base + slot * STB, base + (slot ^ 1) * STB, fo, acc);
}

// ---------------------------------------------------------------------------
// Epilogue staging: a lane's four results of tile (i, j) are four
// consecutive features of one token row: one 8-byte LDS write as bf16.
// ---------------------------------------------------------------------------
template <int COLS>
constexpr int ep_stride() { return COLS * 2 + 32; }

template <int NI, int NJ, int S, class V>
__device__ __forceinline__ void stage4(lds_t* t, int row0, int col0, V v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = row0 + i * 16 + (lane & 15);
      const int col = col0 + j * 16 + 4 * (lane >> 4);
      u32x2_t w;
      w[0] = pack_bf16x2(v(i, j, 0), v(i, j, 1));
      w[1] = pack_bf16x2(v(i, j, 2), v(i, j, 3));
      *(__attribute__((address_space(3))) u32x2_t*)(t + row * S + col * 2) = w;
    }
}

template <int ROWS, int COLS, int S>
__device__ __forceinline__ void lds_to_global(const lds_t* t, bf16_t* C, int64_t ldc, int row_lim,
                                              int col_lim) {
  constexpr int CPR = COLS / 8;
#pragma unroll 4
  for (int q = threadIdx.x; q < ROWS * CPR; q += NTHR) {
    const int row = q / CPR, c8 = q % CPR;
    if (row < row_lim && c8 * 8 < col_lim)  // streamed out: no L2 line kept for the output
      __builtin_nontemporal_store(*(const __attribute__((address_space(3))) u32x4_t*)(t + row * S + c8 * 16),
                                  (u32x4_t*)(C + (int64_t)row * ldc + c8 * 8));
  }
}

template <int ROWS>
__device__ __forceinline__ void load_row_weights(lds_f32_t* wl, const float* topk_w,
                                                 const int32_t* src_of, int m0, int seg1) {
  for (int t = threadIdx.x; t < ROWS; t += NTHR) {
    const int row = m0 + t;
    wl[t] = row < seg1 ? topk_w[src_of[row]] : 0.0f;
  }
}

// ===========================================================================
// Ragged-row GEMMs: token rows are an expert's segment of the sorted rows.
// ===========================================================================
// EPI_STORE: bf16 result; EPI_GATEUP: SwiGLU and top-k weight; EPI_STORE_F32:
// fp32 result (the down dgrad's G, which the SwiGLU backward re-encodes, so
// it is not rounded to bf16 on the way).
enum Epi { EPI_STORE = 0, EPI_GATEUP = 1, EPI_STORE_F32 = 2 };

struct Rows8Args {
  // token side: row r reads A + arow(r) * lda, arow = a_src ? a_src[r] / a_div : r;
  // its scale word at K step kb is As[srow * a_srow + kb * a_skb], srow = r
  // (a_s_sorted: words stored per expert-sorted row, also for gathered token
  // rows) or arow; run-major words (a_srow = 1) put one K step's words of
  // consecutive rows side by side
  const uint8_t* A;
  int64_t lda;
  const int32_t* a_src;
  int a_div;
  const uint32_t* As;
  int64_t a_srow, a_skb;
  int a_s_sorted;
  // feature side (expert e): row n reads B + e * b_estride + wrow(n) * ldb,
  // scale word Bs[e * bs_estride + (wrow(n) >> b_rshift) * b_srow + kb * b_skb]
  // (b_rshift 7: one blockwise scale per 128 rows, row-major; 0: MX codes
  // per row, run-major).
  // gateup: 32-row blocks alternate gate rows (even) and up rows (odd).
  const uint8_t* B;
  int64_t b_estride, ldb;
  const uint32_t* Bs;
  int64_t bs_estride, b_srow, b_skb;
  int b_rshift;
  int gateup;
  // b_kn: the feature side is stored along the features instead, element
  // (n, k) at B + e * b_estride + k * ldb + n (blockwise weights in their
  // forward layout, read by a data gradient); b_srow and b_skb step the
  // scale words per 128 features and per K step as above
  int N, K, n_tiles;  // N: output features (gate/up: gate columns I)
  int row_major;      // tile order within an expert (rows_tile_order)
  const int32_t* offsets;
  const int32_t* tile_off;
  const int4* tiles;  // row-tile descriptors {expert, first row, segment end, expert's first tile}
  int E;
  // EPI_STORE: C [R, ldc] bf16; EPI_STORE_F32: Cf [R, ldc] fp32
  bf16_t* C;
  float* Cf;
  int64_t ldc;
  // EPI_GATEUP: H [R,2I] (optional), Aout [R,I] = w_row * silu(g) * u (g, u
  // clamped at lim: +inf for the plain SwiGLU)
  bf16_t* H;
  bf16_t* Aout;
  int I;
  float lim;
  const float* topk_w;
  const int32_t* src_of;
};

// One row tile of ROWS token rows: 256, or 128 / 64 for a segment's last
// tile holding at most that many rows (the waves then take 64 / 32 rows:
// a half / a quarter of the MFMA work and of the token operand).
template <int EPI, int SC, int ROWS, bool KN>
__device__ __forceinline__ void rows8_tile(const Rows8Args& p, char* smem, int nt, int e, int m0, int seg1) {
  constexpr int TMX = ROWS / WM / 16;
  const int seg0 = m0;  // rows past the segment repeat the tile's first row
  const int lane = threadIdx.x & 63;
  const int wm = wave_m(), wn = wave_n();

  auto srt = [&](int row) -> int64_t {  // expert-sorted row of tile row `row`
    const int r = m0 + row;
    return r < seg1 ? r : seg0;  // rows past the segment: computed, never stored
  };
  auto arow = [&](int row) -> int64_t {
    const int64_t r = srt(row);
    return p.a_src ? (int64_t)(p.a_src[r] / p.a_div) : r;
  };
  auto wrow = [&](int n) -> int {
    if (p.gateup) {
      const int blk = n >> 5;
      int gc = nt * (TBN / 2) + (blk >> 1) * 32 + (n & 31);
      if (gc >= p.I) gc = 0;
      return (blk & 1) ? p.I + gc : gc;
    }
    const int w = nt * TBN + n;
    return w < p.N ? w : 0;
  };
  const uint8_t* Be = p.B + (int64_t)e * p.b_estride;
  const uint32_t* Bse = p.Bs + (int64_t)e * p.bs_estride;
  Op8<ROWS / 64> ot;
  ot.init([&](int row) { return p.A + arow(row) * p.lda; });
  std::conditional_t<KN, Op8KN, Op8<>> of;
  if constexpr (KN) of.init(Be + nt * TBN, p.ldb, p.N - nt * TBN);
  else of.init([&](int n) { return Be + (int64_t)wrow(n) * p.ldb; });
  const int srow = 64 * (wave_id() & 3) + lane;
  const uint32_t* sp = wave_id() < 4 ? p.As + (p.a_s_sorted ? srt(srow) : arow(srow)) * p.a_srow
                                     : Bse + (int64_t)(wrow(srow) >> p.b_rshift) * p.b_srow;
  f32x4_t acc[TMX][TN];
  mainloop8<SC, TMX>(ot, of, sp, (int)(wave_id() < 4 ? p.a_skb : p.b_skb), p.K / KB, smem, acc);

  // ------------------------------------------------------------- epilogues
  barrier_lds();
  lds_t* const lds = (lds_t*)smem;
  const int rows_valid = seg1 - m0;
  const int r0w = wm * (ROWS / WM);
  if constexpr (EPI == EPI_STORE) {
    constexpr int S = ep_stride<TBN>();
    stage4<TMX, TN, S>(lds, r0w, wn * (TBN / WN), [&](int i, int j, int r) { return acc[i][j][r]; });
    barrier_lds();
    lds_to_global<ROWS, TBN, S>(lds, p.C + (int64_t)m0 * p.ldc + nt * TBN, p.ldc, rows_valid,
                                p.N - nt * TBN);
  } else if constexpr (EPI == EPI_STORE_F32) {
    // two passes of 128 columns (the waves with wn = 2h, 2h + 1), 528-byte
    // LDS rows so that a lane group's 16 rows hit distinct banks
    constexpr int SF = 128 * 4 + 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h) barrier_lds();
      if ((wn >> 1) == h) {
#pragma unroll
        for (int i = 0; i < TMX; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int row = r0w + i * 16 + (lane & 15);
            const int col = (wn & 1) * 64 + j * 16 + 4 * (lane >> 4);
            *(__attribute__((address_space(3))) f32x4_t*)(lds + row * SF + col * 4) = acc[i][j];
          }
      }
      barrier_lds();
      float* Cb = p.Cf + (int64_t)m0 * p.ldc + nt * TBN + 128 * h;
      const int col_lim = p.N - nt * TBN - 128 * h;
#pragma unroll 4
      for (int q = threadIdx.x; q < ROWS * 32; q += NTHR) {
        const int row = q >> 5, c4 = q & 31;
        if (row < rows_valid && c4 * 4 < col_lim)
          __builtin_nontemporal_store(*(const __attribute__((address_space(3))) f32x4_t*)(lds + row * SF + c4 * 16),
                                      (f32x4_t*)(Cb + (int64_t)row * p.ldc + c4 * 4));
      }
    }
  } else if constexpr (EPI == EPI_GATEUP) {
    // features j = 0, 1 are gate columns wn*32 + 16 j + ..., j = 2, 3 the up
    // columns of the same gate columns
    constexpr int S = ep_stride<TBN / 2>();
    constexpr int TB = ROWS * S;
    lds_f32_t* wl = (lds_f32_t*)(lds + 2 * TB);
    load_row_weights<ROWS>(wl, p.topk_w, p.src_of, m0, seg1);
    barrier_lds();
    const int c0w = wn * 32;
    stage4<TMX, 2, S>(lds, r0w, c0w, [&](int i, int j, int r) {
      const float g = clamp_gate(acc[i][j][r], p.lim), u = clamp_up(acc[i][j + 2][r], p.lim);
      return wl[r0w + i * 16 + (lane & 15)] * (g * sigmoidf_(g) * u);
    });
    if (p.H) stage4<TMX, 2, S>(lds + TB, r0w, c0w, [&](int i, int j, int r) { return acc[i][j][r]; });
    barrier_lds();
    const int gc0 = nt * (TBN / 2);
    lds_to_global<ROWS, TBN / 2, S>(lds, p.Aout + (int64_t)m0 * p.I + gc0, p.I, rows_valid, p.I - gc0);
    if (p.H) {
      bf16_t* H0 = p.H + (int64_t)m0 * 2 * p.I + gc0;
      lds_to_global<ROWS, TBN / 2, S>(lds + TB, H0, 2 * p.I, rows_valid, p.I - gc0);
      barrier_lds();
      stage4<TMX, 2, S>(lds, r0w, c0w, [&](int i, int j, int r) { return acc[i][j + 2][r]; });
      barrier_lds();
      lds_to_global<ROWS, TBN / 2, S>(lds, H0 + p.I, 2 * p.I, rows_valid, p.I - gc0);
    }
  }
}

// TAG only tells launch sites with the same epilogue apart in profiles.
// SC: SC_WEIGHT (blockwise) or SC_MX.
template <int EPI, int TAG, int SC, bool KN>
__global__ __launch_bounds__(NTHR, 1) void rows8_kernel(Rows8Args p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int L = xcd_tile(blockIdx.x, p.tile_off[p.E] * p.n_tiles);
  if (L < 0) return;
  // An expert's (row tile, N tile) pairs are a contiguous range of L, taken
  // N-tile-major (work-groups that start close together share a weight tile
  // through L2) or, with row_major, row-tile-major (they share token rows);
  // the descriptor of L's row-tile-major row tile lies in the same expert
  // and gives the range.
  const int T = L / p.n_tiles;
  const int4 d0 = p.tiles[T];  // {expert, first row, segment end, expert's first tile}
  const int e = d0.x, seg1 = d0.z, first = d0.w;
  const int seg0 = d0.y - (T - first) * TBM;
  const int nrt = (seg1 - seg0 + TBM - 1) / TBM;
  const int j = L - first * p.n_tiles;
  const int rt = p.row_major ? j / p.n_tiles : j % nrt;
  const int nt = p.row_major ? j - rt * p.n_tiles : j / nrt;
  const int m0 = seg0 + rt * TBM;
  const int rows = seg1 - m0;
  if (rows <= TBM / 4) rows8_tile<EPI, SC, TBM / 4, KN>(p, smem, nt, e, m0, seg1);
  else if (rows <= TBM / 2) rows8_tile<EPI, SC, TBM / 2, KN>(p, smem, nt, e, m0, seg1);
  else rows8_tile<EPI, SC, TBM, KN>(p, smem, nt, e, m0, seg1);
}

// ===========================================================================
// Weight gradients: dW[e][m, n] = sum over expert e's token blocks of
// A(m, k) B(n, k) s_A(m, blk) s_B(n, blk).  Both operands are transposed
// token-blocked ([features][padded rows], see quant_fp8.hip): expert e owns
// K bytes [128 blk_off[e], 128 blk_off[e+1]) of every row, and one scale
// word per row and 128-row run, stored run-major so that a K step's words
// for 256 consecutive rows are one contiguous kilobyte.
// ===========================================================================
struct Wgrad8Args {
  const uint8_t* A;    // output-row side, [M][ldk]
  const uint32_t* As;  // [run][M]
  const uint8_t* B;    // output-column side, [N][ldk]
  const uint32_t* Bs;  // [run][N]
  int64_t ldk;
  int M, N, m_tiles, n_tiles, E;
  const int32_t* blk_off;
  const int32_t* xorder;  // expert of each (slot, XCD): see the schedule
  bf16_t* C;  // dW[e] = C + e * c_estride, row-major [M, N]
  int64_t c_estride;
};

// SC: SC_ROW (blockwise) or SC_MX.
template <int TAG, int SC>
__global__ __launch_bounds__(NTHR, 1) void wgrad8_kernel(Wgrad8Args p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int per = p.m_tiles * p.n_tiles;
  const int slot = (blockIdx.x >> 3) / per;  // the work-group runs on XCD blockIdx.x % 8
  if (slot >= (p.E + 7) / 8) return;
  const int e = p.xorder[slot * 8 + (blockIdx.x & 7)];
  if (e < 0) return;
  const int rem = (blockIdx.x >> 3) % per;
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int b0 = p.blk_off[e];
  const int nkb = p.blk_off[e + 1] - b0;
  auto mrow = [&](int row) { const int m = mt * TBM + row; return m < p.M ? m : 0; };
  auto nrow = [&](int row) { const int n = nt * TBN + row; return n < p.N ? n : 0; };
  Op8<> ot, of;
  ot.init([&](int row) { return p.A + (int64_t)mrow(row) * p.ldk + (int64_t)b0 * KB; });
  of.init([&](int row) { return p.B + (int64_t)nrow(row) * p.ldk + (int64_t)b0 * KB; });
  const int srow = 64 * (wave_id() & 3) + (threadIdx.x & 63);
  const uint32_t* sp = wave_id() < 4 ? p.As + (int64_t)b0 * p.M + mrow(srow) : p.Bs + (int64_t)b0 * p.N + nrow(srow);
  f32x4_t acc[TM][TN];
  mainloop8<SC, TM>(ot, of, sp, wave_id() < 4 ? p.M : p.N, nkb, smem, acc);
  barrier_lds();
  lds_t* const lds = (lds_t*)smem;
  constexpr int S = ep_stride<TBN>();
  stage4<TM, TN, S>(lds, wave_m() * (TBM / WM), wave_n() * (TBN / WN),
                    [&](int i, int j, int r) { return acc[i][j][r]; });
  barrier_lds();
  lds_to_global<TBM, TBN, S>(lds, p.C + (int64_t)e * p.c_estride + (int64_t)mt * TBM * p.N + nt * TBN,
                             p.N, p.M - mt * TBM, p.N - nt * TBN);
}

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t kRingBytes = (size_t)2 * STB;
constexpr size_t kStoreEpi = (size_t)TBM * ep_stride<TBN>();
constexpr size_t kGateupEpi = (size_t)2 * TBM * ep_stride<TBN / 2>() + TBM * 4;
constexpr size_t kStoreF32Epi = (size_t)TBM * (128 * 4 + 16);
constexpr size_t kSmem = cmax(cmax(kRingBytes, kStoreF32Epi), cmax(kStoreEpi, kGateupEpi));
static_assert(kSmem <= 160 * 1024, "LDS");

template <int EPI, int TAG, int SC, bool KN = false>
hipError_t launch_rows8_sc(const LaunchCtx& c, const char* name, const Rows8Args& p, int R) {
  {
    hipError_t e = allow_smem_once<rows8_kernel<EPI, TAG, SC, KN>>(kSmem);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (int64_t)(R / TBM + p.E) * p.n_tiles;
  const unsigned nblocks = (unsigned)((tiles + 7) / 8 * 8);
  MOE_LAUNCH(c, name, (rows8_kernel<EPI, TAG, SC, KN>), dim3(nblocks), dim3(NTHR), kSmem, p);
  return hipSuccess;
}

// kn: the feature side in its forward layout (blockwise weights only)
template <int EPI, int TAG>
hipError_t launch_rows8(const LaunchCtx& c, const char* name, Rows8Args p, int R, bool mx, bool kn = false) {
  p.b_rshift = mx ? 0 : 7;
  if (mx) return launch_rows8_sc<EPI, TAG, SC_MX>(c, name, p, R);
  return kn ? launch_rows8_sc<EPI, TAG, SC_WEIGHT, true>(c, name, p, R)
            : launch_rows8_sc<EPI, TAG, SC_WEIGHT>(c, name, p, R);
}

template <int TAG, int SC>
hipError_t launch_wgrad8_sc(const LaunchCtx& c, const char* name, const Wgrad8Args& p) {
  {
    hipError_t e = allow_smem_once<wgrad8_kernel<TAG, SC>>(kSmem);
    if (e != hipSuccess) return e;
  }
  const unsigned nblocks = (unsigned)(cdiv(p.E, 8) * 8 * p.m_tiles * p.n_tiles);
  MOE_LAUNCH(c, name, (wgrad8_kernel<TAG, SC>), dim3(nblocks), dim3(NTHR), kSmem, p);
  return hipSuccess;
}

template <int TAG>
hipError_t launch_wgrad8(const LaunchCtx& c, const char* name, const Wgrad8Args& p, bool mx) {
  return mx ? launch_wgrad8_sc<TAG, SC_MX>(c, name, p) : launch_wgrad8_sc<TAG, SC_ROW>(c, name, p);
}

}  // namespace

int fp8_dw_blocks(int I) { return I / 128; }  // one partial per 128 columns of I

namespace {
// Scale words per expert of a weight [N, K] encoded for a GEMM with K along
// its rows: blockwise (N/128) x (K/128) fp32 scales (row-major), MX N x K/32
// codes (words run-major, [K/128][N]).
int64_t wscale_words(int64_t N, int64_t K, bool mx) { return (mx ? N : N / 128) * (K / 128); }

hipError_t quant_weights(const LaunchCtx& c, const char* name, const void* W, int E, int N, int K,
                         bool mx, uint8_t* q, void* s, uint8_t* qt, void* st) {
  if (mx)  // run-major words: one K step's words of consecutive rows are contiguous
    return launch_quant_weight_mx(c, name, W, E, N, K, q, (uint8_t*)s, qt, (uint8_t*)st, true);
  return launch_quant_weight(c, name, W, E, N, K, q, (float*)s, qt, (float*)st);
}
}  // namespace

hipError_t fp8_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Fwd& q, void* H, void* Aw,
                         void* Yw) {
  const int64_t I = a.I, d = a.d;
  const bool mx = q.mx;
  // x's scale words per expert-sorted row (run-major), so that the gathering
  // gate/up GEMM reads one K step's words contiguously
  HIP_RET(launch_quant_rows(c, "quant_x", a.x, d, a.T, a.d, q.xq, q.xs, mx, true, a.row_of, a.k));
  // The backward's data gradients contract over the weights' other axis.
  // Blockwise, a 128 x 128 block has one scale either way, so they read the
  // forward codes along the weight rows: those go straight into `saved` when
  // it is kept.  MX blocks run along one axis: a second, transposed encoding
  // (from the same read) goes into `saved`.
  uint8_t* wguq = q.wguq; void* wgus = q.wgus;
  uint8_t* wdq = q.wdq; void* wds = q.wds;
  if (!mx && q.sv.wgu_dgq) { wguq = q.sv.wgu_dgq; wgus = q.sv.wgu_dgs; }
  if (!mx && q.sv.wd_dgq) { wdq = q.sv.wd_dgq; wds = q.sv.wd_dgs; }
  HIP_RET(quant_weights(c, "quant_w_gate_up", a.w_gate_up, a.E, 2 * a.I, a.d, mx, wguq, wgus,
                        mx ? q.sv.wgu_dgq : nullptr, mx ? q.sv.wgu_dgs : nullptr));
  if (wdq || (mx && q.sv.wd_dgq))
    HIP_RET(quant_weights(c, "quant_w_down", a.w_down, a.E, a.d, a.I, mx, wdq, wds,
                          mx ? q.sv.wd_dgq : nullptr, mx ? q.sv.wd_dgs : nullptr));
  {  // gate/up GEMM on token rows gathered from xq; SwiGLU and top-k weight in the epilogue
    Rows8Args p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = q.xq; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.As = (const uint32_t*)q.xs; p.a_srow = 1; p.a_skb = a.R; p.a_s_sorted = 1;
    p.B = wguq; p.b_estride = 2 * I * d; p.ldb = d;
    p.Bs = (const uint32_t*)wgus; p.bs_estride = wscale_words(2 * I, d, mx);
    p.b_srow = mx ? 1 : d / 128; p.b_skb = mx ? 2 * I : 1;
    p.gateup = 1;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, TBN / 2);
    p.row_major = rows_tile_order(a.T * d, a.E * 2 * I * d);
    p.H = (bf16_t*)H; p.Aout = (bf16_t*)Aw; p.I = a.I; p.lim = a.swiglu_lim;
    p.topk_w = a.topk_w; p.src_of = a.src_of;
    HIP_RET(launch_rows8<EPI_GATEUP, 0>(c, "gemm_gateup_fwd", p, a.R, mx));
  }
  if (!Yw) return hipSuccess;  // the gate/up half alone (recomputation)
  HIP_RET(launch_quant_rows(c, "quant_aw", Aw, I, a.R, a.I, q.awq, q.aws, mx, true));
  Rows8Args p = {};  // down GEMM: Yw = Aw W_down[e]^T
  p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
  p.A = q.awq; p.lda = I; p.a_src = nullptr; p.a_div = 1;
  p.As = (const uint32_t*)q.aws; p.a_srow = 1; p.a_skb = a.R;
  p.B = wdq; p.b_estride = d * I; p.ldb = I;
  p.Bs = (const uint32_t*)wds; p.bs_estride = wscale_words(d, I, mx);
  p.b_srow = mx ? 1 : I / 128; p.b_skb = mx ? d : 1;
  p.gateup = 0;
  p.N = a.d; p.K = a.I; p.n_tiles = (int)cdiv(a.d, TBN);
  p.row_major = rows_tile_order(a.R * I, a.E * d * I);
  p.C = (bf16_t*)Yw; p.ldc = d;
  return launch_rows8<EPI_STORE, 0>(c, "gemm_down_fwd", p, a.R, mx);
}

hipError_t fp8_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Bwd& q, const void* dout,
                         const void* H, const void* Aw, void* dXp, float* dwp, void* dW_gu, void* dW_d) {
  const int64_t I = a.I, d = a.d;
  const bool mx = q.mx;
  if (q.quant_weights) {  // the data gradients' encodings only (see fp8_fwd_gemms)
    HIP_RET(quant_weights(c, "quant_w_gate_up", a.w_gate_up, a.E, 2 * a.I, a.d, mx, mx ? nullptr : q.sv.wgu_dgq,
                          mx ? nullptr : q.sv.wgu_dgs, mx ? q.sv.wgu_dgq : nullptr, mx ? q.sv.wgu_dgs : nullptr));
    HIP_RET(quant_weights(c, "quant_w_down", a.w_down, a.E, a.d, a.I, mx, mx ? nullptr : q.sv.wd_dgq,
                          mx ? nullptr : q.sv.wd_dgs, mx ? q.sv.wd_dgq : nullptr, mx ? q.sv.wd_dgs : nullptr));
  }
  HIP_RET(launch_quant_rows(c, "quant_dout", dout, d, a.T, a.d, q.doutq, q.douts, mx, true, a.row_of, a.k));
  {  // down dgrad: G = dout_t W_down[e] (fp32)
    Rows8Args p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = q.doutq; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.As = (const uint32_t*)q.douts; p.a_srow = 1; p.a_skb = a.R; p.a_s_sorted = 1;
    p.B = q.sv.wd_dgq; p.b_estride = I * d;
    p.Bs = (const uint32_t*)q.sv.wd_dgs; p.bs_estride = wscale_words(I, d, mx);
    if (mx) {  // transposed codes [E,I,d], rows along I
      p.ldb = d; p.b_srow = 1; p.b_skb = I;
    } else {   // forward codes [E,d,I] read along I; scales [d/128][I/128]
      p.ldb = I; p.b_srow = 1; p.b_skb = I / 128;
    }
    p.gateup = 0;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, TBN);
    p.row_major = rows_tile_order(a.T * d, a.E * d * I);
    p.Cf = q.G; p.ldc = I;
    HIP_RET(launch_rows8<EPI_STORE_F32, 2>(c, "gemm_down_dgrad", p, a.R, mx, !mx));
  }
  const int nb = q.nblk_max;
  {  // down wgrad: dW_d[e][c, i] = sum_r dout[t_r, c] Aw[r, i]
    HIP_RET(launch_quant_tok(c, "quant_dout_tok", dout, d, a.src_of, a.k, a.d, a.offsets, q.blk_off,
                             a.E, nb, q.tqa, q.tsa, mx, true));
    HIP_RET(launch_quant_tok(c, "quant_aw_tok", Aw, I, nullptr, 1, a.I, a.offsets, q.blk_off, a.E, nb,
                             q.tqb, q.tsb, mx, true));
    Wgrad8Args p = {};
    p.A = q.tqa; p.As = (const uint32_t*)q.tsa; p.B = q.tqb; p.Bs = (const uint32_t*)q.tsb;
    p.ldk = (int64_t)nb * KB;
    p.M = a.d; p.N = a.I; p.m_tiles = (int)cdiv(a.d, TBM); p.n_tiles = (int)cdiv(a.I, TBN); p.E = a.E;
    p.blk_off = q.blk_off; p.xorder = a.xorder;
    p.C = (bf16_t*)dW_d; p.c_estride = d * I;
    HIP_RET(launch_wgrad8<0>(c, "gemm_down_wgrad", p, mx));
  }
  // SwiGLU backward from G: dH never leaves the kernel; its row codes feed
  // the gate/up dgrad and its token-block codes (into tqa, free once the
  // down wgrad has run) the gate/up wgrad
  HIP_RET(launch_swiglu_bwd_tok(c, q.G, H, a.topk_w, a.src_of, a.R, a.I, a.swiglu_lim, a.offsets, q.blk_off,
                                a.E, nb, dwp, q.dhq, q.dhs, q.tqa, q.tsa, mx));
  {  // gate/up dgrad: dXp = dH W_gate_up[e]
    Rows8Args p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = q.dhq; p.lda = 2 * I; p.a_src = nullptr; p.a_div = 1;
    p.As = (const uint32_t*)q.dhs; p.a_srow = 1; p.a_skb = a.R;  // run-major
    p.B = q.sv.wgu_dgq; p.b_estride = d * 2 * I;
    p.Bs = (const uint32_t*)q.sv.wgu_dgs; p.bs_estride = wscale_words(d, 2 * I, mx);
    if (mx) {  // transposed codes [E,d,2I], rows along d
      p.ldb = 2 * I; p.b_srow = 1; p.b_skb = d;
    } else {   // forward codes [E,2I,d] read along d; scales [2I/128][d/128]
      p.ldb = d; p.b_srow = 1; p.b_skb = d / 128;
    }
    p.gateup = 0;
    p.N = a.d; p.K = 2 * a.I; p.n_tiles = (int)cdiv(a.d, TBN);
    p.row_major = rows_tile_order(a.R * 2 * I, a.E * 2 * I * d);
    p.C = (bf16_t*)dXp; p.ldc = d;
    HIP_RET(launch_rows8<EPI_STORE, 1>(c, "gemm_gateup_dgrad", p, a.R, mx, !mx));
  }
  {  // gate/up wgrad: dW_gu[e][j, c] = sum_r dH[r, j] x[t_r, c]
    HIP_RET(launch_quant_tok(c, "quant_x_tok", a.x, d, a.src_of, a.k, a.d, a.offsets, q.blk_off, a.E,
                             nb, q.tqb, q.tsb, mx, true));
    Wgrad8Args p = {};
    p.A = q.tqa; p.As = (const uint32_t*)q.tsa; p.B = q.tqb; p.Bs = (const uint32_t*)q.tsb;
    p.ldk = (int64_t)nb * KB;
    p.M = 2 * a.I; p.N = a.d; p.m_tiles = (int)cdiv(2 * a.I, TBM); p.n_tiles = (int)cdiv(a.d, TBN);
    p.E = a.E; p.blk_off = q.blk_off; p.xorder = a.xorder;
    p.C = (bf16_t*)dW_gu; p.c_estride = 2 * I * d;
    HIP_RET(launch_wgrad8<1>(c, "gemm_gateup_wgrad", p, mx));
  }
  return hipSuccess;
}

}  // namespace moe
