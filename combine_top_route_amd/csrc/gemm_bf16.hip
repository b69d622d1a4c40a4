// Grouped GEMMs of the expert MLPs in bf16 on gfx950 MFMA (fp32 accumulate).
//
// Each expert is a SwiGLU MLP: both expert linear layers plus SwiGLU
// ("Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed", section
// "What a mixture-of-experts layer actually does"; "Mario/overlap moe kernel
// integration", overview: "SwiGLU expert GEMMs").  Fusion keeps
// intermediates out of separate passes ("Prime Intellect's Prime Mega MoE
// Trains Giant AI Models 55% Faster", section "One kernel overlaps the
// pipeline"): the token gather is the A-operand load of the gate/up GEMM,
// and SwiGLU and the top-k weighting are its epilogue.  (The SwiGLU backward
// is a separate row pass after the down dgrad: fused into that epilogue it
// cost more than the HBM traffic it saved.)
//
// Tile engine (all six GEMMs): C[m,n] = sum_k A(m,k) B(n,k) on a 256x256
// output tile, K in steps of 64, eight waves (two per SIMD) of 128x64, each
// 4x2 MFMA 32x32x16 bf16 tiles: the largest tile whose accumulators (128
// per lane) fit the registers at two waves per SIMD.  A 256x256x64 step
// moves 64 KB per 2048 MFMA cycles; that stream (its L2 misses, and the LDS
// that the direct loads share with the fragment reads) is what bounds the
// main loop.  Operands move global -> LDS with direct loads
// (global_load_lds_dwordx4, no register staging) into a ring: two 64 KB
// stages for the gradients, whose loads of step k+1 all leave at the start
// of step k, and five 32 KB half stages for the forward GEMMs (weights two
// steps ahead, token rows one).  For the gate/up GEMM the loads in flight are
// the gathered token rows of the next K slice, the one-GPU analogue of
// computing on one token group while the next one moves.  One barrier per K
// step.
//
// LDS layouts: an operand whose rows are K-contiguous in memory is stored
// [row][64 k] and read with ds_read_b128; an operand whose rows are contiguous
// along M/N (the weights in the dgrads, both operands of the weight
// gradients) is stored [k][cols] and read with ds_read_b64_tr_b16, whose
// 16-lane transpose hands each lane four consecutive k of one column.  Both
// layouts are XOR-swizzled so the reads of one instruction hit distinct
// banks.
#include "common.h"
#include "tile.h"

#include <algorithm>

namespace moe {
namespace {
using namespace tile;

constexpr int BK = 64;
constexpr int NSTAGE = 2;
constexpr int NWAVE = 8;
constexpr int NTHR = NWAVE * 64;
constexpr int WM = 2, WN = 4;          // wave grid
constexpr int TBM = 256, TBN = 256;    // output tile
constexpr int TM = TBM / WM / 32;      // MFMA tiles per wave along M (4)
constexpr int TN = TBN / WN / 32;      // MFMA tiles per wave along N (2)
static_assert(TBM == kRowTile, "tile table is built for 256-row tiles");

// Source of the direct loads that fall outside an operand (K tail, columns
// past N, rows past an expert's segment in the weight gradients).
__device__ __attribute__((aligned(64))) uint8_t g_zero_page[64] = {0};

// [k][cols] layout: 32-byte chunks XOR-swizzled by k-row so that the four
// rows read together by a 16-lane group, and the two column halves of a
// 32-column fragment, land in distinct bank ranges.
__device__ __forceinline__ int km_swz(int krow) { return ((krow & 3) << 1) ^ ((krow >> 1) & 1); }

// ---------------------------------------------------------------------------
// Operand with K-contiguous rows (row r at rowp(r), element k at rowp(r)[k]).
// ROWS x 64 tile; instruction q covers rows 8q..8q+7 (1 KB of LDS); wave w
// issues q = w, w+8, ...  Each lane keeps one global pointer per instruction,
// advanced by 64 elements per K step; only a partial last K step checks
// bounds.
// ---------------------------------------------------------------------------
template <int ROWS>
struct OpMK {
  static constexpr bool TR = false;  // fragments read with plain ds_read_b128
  static constexpr bool GATHERED = false;
  static constexpr int NI = ROWS * BK * 2 / 1024 / NWAVE;
  static constexpr int BYTES = ROWS * BK * 2;
  const bf16_t* ptr[NI];  // address of this lane's chunk at the current K step
  int K;

  // element offset inside a K step of this lane's chunk in instruction i
  __device__ static int koff(int i) {
    const int lane = threadIdx.x & 63;
    const int row = 8 * ((threadIdx.x >> 6) + NWAVE * i) + (lane >> 3);
    return ((lane & 7) ^ mk_swz(row)) << 3;
  }
  // tile row of this lane's chunk in instruction i
  __device__ static int lane_row(int i) { return 8 * ((threadIdx.x >> 6) + NWAVE * i) + ((threadIdx.x & 63) >> 3); }
  // rowp_of(i, row): the address of tile row `row`, which instruction i loads
  template <class F>
  __device__ void init(F rowp_of, int K_) {
    K = K_;
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] = rowp_of(i, lane_row(i)) + koff(i);
  }
  // number of leading K steps (of nk) that need no bounds checks
  __device__ int nfull(int nk) const { return K / BK < nk ? K / BK : nk; }
  template <int I0, int I1, bool FULL>
  __device__ void issue(int kt, lds_t* s) const {
    const int w = wave_id();
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const void* g = ptr[i];
      if constexpr (!FULL) {
        if (kt * BK + koff(i) >= K) g = g_zero_page;
      }
      dma16(g, s + (w + NWAVE * i) * 1024);
    }
  }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] += BK;
  }
  __device__ static bf16x8_t frag(const lds_t* s, int rb, int kk) {
    const int lane = threadIdx.x & 63;
    const int row = rb + (lane & 31);
    return *(const __attribute__((address_space(3))) bf16x8_t*)(s + mk_off(row, kk * 2 + (lane >> 5)));
  }
};

// ---------------------------------------------------------------------------
// Operand with column-contiguous k-rows: element (col, k) = base[k * ld + col]
// for k < KR (rows past KR read as zero).  COLS x 64 tile stored [k][COLS];
// instruction q covers k-rows q*RPI..  Columns at or past N read as zero.
// ---------------------------------------------------------------------------
template <int COLS>
struct OpKM {
  static constexpr bool TR = true;          // fragments read with ds_read_b64_tr_b16
  static constexpr bool GATHERED = false;
  static constexpr int RB = COLS * 2;       // bytes per k-row
  static constexpr int UPR = RB / 16;       // 16-byte units per k-row
  static constexpr int RPI = 1024 / RB;     // k-rows per instruction
  static constexpr int NI = BK / RPI / NWAVE;
  static constexpr int BYTES = COLS * BK * 2;
  const bf16_t* ptr[NI];  // address at the current K step (not dereferenced when outside)
  int64_t step;           // elements per K step (64 * ld)
  int c0, KR, N;
  bool cfull;             // the tile's columns all lie inside N

  // k-row (0..63) and tile column of this lane's 16-byte unit in instruction i
  __device__ static int krow(int i) {
    return ((threadIdx.x >> 6) + NWAVE * i) * RPI + (threadIdx.x & 63) / UPR;
  }
  __device__ static int ucol(int i) {
    const int p = (threadIdx.x & 63) % UPR;
    return ((((p >> 1) ^ km_swz(krow(i))) << 1) | (p & 1)) * 8;
  }
  __device__ void init(const bf16_t* base, int64_t ld, int c0_, int N_, int KR_) {
    c0 = c0_;
    KR = KR_;
    N = N_;
    cfull = c0_ + COLS <= N_;
    step = (int64_t)BK * ld;
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] = base + (int64_t)krow(i) * ld + c0_ + ucol(i);
  }
  __device__ int nfull(int nk) const { return !cfull ? 0 : (KR / BK < nk ? KR / BK : nk); }
  template <int I0, int I1, bool FULL>
  __device__ void issue(int kt, lds_t* s) const {
    const int w = wave_id();
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const void* g = ptr[i];
      if constexpr (!FULL) {
        if (kt * BK + krow(i) >= KR || c0 + ucol(i) >= N) g = g_zero_page;
      }
      dma16(g, s + (w + NWAVE * i) * 1024);
    }
  }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < NI; ++i) ptr[i] += step;
  }
  __device__ static bf16x8_t frag(const lds_t* s, int cb, int kk) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, sl = lane & 15;
    const int col = cb + (g & 1) * 16 + 4 * (sl & 3);
    const int kr0 = kk * 16 + (g >> 1) * 8 + (sl >> 2);
    const int kr1 = kr0 + 4;
    const int ch = col >> 4;
    const lds_t* p0 = s + kr0 * RB + ((ch ^ km_swz(kr0)) << 5) + ((col & 15) << 1);
    const lds_t* p1 = s + kr1 * RB + ((ch ^ km_swz(kr1)) << 5) + ((col & 15) << 1);
    s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p0);
    s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p1);
    s16x8_t c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, c);
  }
};

// ---------------------------------------------------------------------------
// Column-contiguous operand whose k-rows are rows of an expert's segment:
// element (col, k) = base[row(seg0 + k) * ld + col] for k < KR, with
// row(r) = tok[r] (GATHER: the token of row r, a row of x or dout) or r.
// The row indices of the next stage to issue are formed one K step ahead.
// ---------------------------------------------------------------------------
template <int COLS, bool GATHER>
struct OpKMg {
  static constexpr bool TR = true;
  static constexpr bool GATHERED = GATHER;  // stage addresses come from loaded row indices
  static constexpr int RB = COLS * 2;
  static constexpr int UPR = RB / 16;
  static constexpr int RPI = 1024 / RB;
  static constexpr int NI = BK / RPI / NWAVE;
  static constexpr int BYTES = COLS * BK * 2;
  const bf16_t* base;
  int64_t ld;
  const int32_t* tok;
  int seg0, c0, KR, N;
  int nkt;         // stage whose rows are in nrow[]
  int nrow[NI];    // row of this lane's k-row in instruction i for stage nkt
  unsigned nmask;  // bit i: that k-row lies inside the segment
  bool cfull;

  __device__ static int krow(int i) {
    return ((threadIdx.x >> 6) + NWAVE * i) * RPI + (threadIdx.x & 63) / UPR;
  }
  __device__ static int ucol(int i) {
    const int p = (threadIdx.x & 63) % UPR;
    return ((((p >> 1) ^ km_swz(krow(i))) << 1) | (p & 1)) * 8;
  }
  // The token loads are unconditional (k-rows past the segment read a row
  // inside it, or row 0 of an empty segment) and nothing consumes their
  // values before the next stage is issued, one K step later, after that
  // step's wait: a load under a branch, or a select on its value, would make
  // the compiler wait for every load in flight, the stage just issued
  // included.
  __device__ void fetch_rows(int kt) {
    nkt = kt;
    nmask = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = kt * BK + krow(i);
      const bool in = k < KR;
      nmask |= (unsigned)in << i;
      if constexpr (GATHER) nrow[i] = tok[KR > 0 ? seg0 + (in ? k : KR - 1) : 0];
      else nrow[i] = seg0 + k;
    }
  }
  __device__ void init(const bf16_t* base_, int64_t ld_, const int32_t* tok_, int seg0_, int c0_, int N_,
                       int KR_) {
    base = base_; ld = ld_; tok = tok_; seg0 = seg0_;
    c0 = c0_; N = N_; KR = KR_;
    cfull = c0_ + COLS <= N_;
    fetch_rows(0);
  }
  __device__ int nfull(int nk) const { return !cfull ? 0 : (KR / BK < nk ? KR / BK : nk); }
  template <int I0, int I1, bool FULL>
  __device__ void issue(int, lds_t* s) const {
    const int w = wave_id();
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int c = c0 + ucol(i);
      const void* g;
      if constexpr (FULL) {  // every k-row of the stage lies in the segment, every column in N
        g = base + (int64_t)nrow[i] * ld + c;
      } else {
        const bool ok = ((nmask >> i) & 1) && c < N;
        g = ok ? (const void*)(base + (int64_t)nrow[i] * ld + c) : (const void*)g_zero_page;
      }
      dma16(g, s + (w + NWAVE * i) * 1024);
    }
  }
  // the stage just issued is done with nrow[]: form the rows of the next one
  __device__ void advance() { fetch_rows(nkt + 1); }
  __device__ static bf16x8_t frag(const lds_t* s, int cb, int kk) { return OpKM<COLS>::frag(s, cb, kk); }
};

// Issues part P (of 4) of a stage's direct loads of operand O (FULL: the
// stage needs no bounds checks).
template <int P, bool FULL, class O>
__device__ __forceinline__ void issue_part(const O& o, int kt, lds_t* s) {
  constexpr int per = (O::NI + 3) / 4;
  constexpr int i0 = P * per < O::NI ? P * per : O::NI;
  constexpr int i1 = (P + 1) * per < O::NI ? (P + 1) * per : O::NI;
  if constexpr (i1 > i0) o.template issue<i0, i1, FULL>(kt, s);
}

template <bool FULL, class OA, class OB>
__device__ __forceinline__ void issue_stage(const OA& oa, const OB& ob, int kt, lds_t* dst) {
  issue_part<0, FULL>(oa, kt, dst); issue_part<0, FULL>(ob, kt, dst + OA::BYTES);
  issue_part<1, FULL>(oa, kt, dst); issue_part<1, FULL>(ob, kt, dst + OA::BYTES);
  issue_part<2, FULL>(oa, kt, dst); issue_part<2, FULL>(ob, kt, dst + OA::BYTES);
  issue_part<3, FULL>(oa, kt, dst); issue_part<3, FULL>(ob, kt, dst + OA::BYTES);
}

// Wave position in the 2 x 4 wave grid.
__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) / WN; }
__device__ __forceinline__ int wave_n() { return (threadIdx.x >> 6) % WN; }

// One K step: wait for this wave's loads of the step, barrier (every wave's
// loads have landed and every wave is done with the slot to be refilled),
// then four 16-k sub-steps, each reading the next sub-step's fragments while
// its MFMAs run.  SS is the byte distance between the ring's two slots (0:
// one stage apart).  IS issues the next stage: IS::early() runs right after
// the barrier, IS::issue(dst) in sub-step IK (the first when IK < 0).
//
// The body takes the slot it reads and the slot the loads fill as
// __restrict__ parameters.  Without that, the compiler cannot tell a
// transposing LDS read (ds_read_b64_tr_b16) apart from the slot that direct
// loads are filling, and makes every such read wait for all direct loads in
// flight; with it, the next stage's loads leave at the start of the step in
// all six GEMMs and have the whole step to land.
template <int TMX, bool PRE, int ISSUE_KK, class OA, class OB, class IS>
__device__ __forceinline__ void kstep_body(IS& is, const lds_t* __restrict__ As, const lds_t* __restrict__ Bs,
                                           lds_t* __restrict__ dst, f32x16_t (&acc)[TMX][TN]) {
  constexpr int NKK = BK / 16;
  const int wm = wave_m(), wn = wave_n();
  if constexpr (PRE) is.early();
  bf16x8_t a[2][TMX], b[2][TN];
#pragma unroll
  for (int i = 0; i < TMX; ++i) a[0][i] = OA::frag(As, wm * (TMX * 32) + i * 32, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) b[0][j] = OB::frag(Bs, wn * (TBN / WN) + j * 32, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int cur = kk & 1;
    // this sub-step's fragments are all in registers before its first MFMA
    // (read during the previous sub-step), so no MFMA below waits on reads
    // issued after it
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (kk + 1 < NKK) {
#pragma unroll
      for (int i = 0; i < TMX; ++i) a[cur ^ 1][i] = OA::frag(As, wm * (TMX * 32) + i * 32, kk + 1);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[cur ^ 1][j] = OB::frag(Bs, wn * (TBN / WN) + j * 32, kk + 1);
    }
    if constexpr (PRE) {
      if (kk == ISSUE_KK) is.issue(dst);
    }
#pragma unroll
    for (int i = 0; i < TMX; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[cur][j], a[cur][i], acc[i][j], 0, 0, 0);
    // one fragment read (and direct load) after each MFMA, so the reads of
    // the next sub-step and the loads of the next stage issue while this
    // sub-step's MFMAs run, and nothing here waits for them
    // (a transposed fragment takes two reads)
    const int NR = (kk + 1 < NKK ? TMX * (OA::TR ? 2 : 1) + TN * (OB::TR ? 2 : 1) : 0);
    const int NG = (PRE && kk == ISSUE_KK) ? OA::NI + OB::NI : 0;
#pragma unroll
    for (int q = 0; q < TMX * TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
      if (q * 2 + 1 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
      else if (q * 2 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < NG) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int TMX, bool PRE, int SS, int IK, class OA, class OB, class IS>
__device__ __forceinline__ void kstep_core(IS& is, lds_t* base, int& slot, f32x16_t (&acc)[TMX][TN]) {
  constexpr int ST = SS ? SS : OA::BYTES + OB::BYTES;
  wait_vmcnt<0>();
  barrier_lds();
  const lds_t* As = base + slot * ST;
  kstep_body<TMX, PRE, (IK >= 0 ? IK : 0), OA, OB>(is, As, As + OA::BYTES, base + (slot ^ 1) * ST, acc);
  slot ^= 1;
}

// The next stage of the tile's own operands.
template <bool FULL, class OA, class OB>
struct SelfIssue {
  const OA& oa;
  const OB& ob;
  int kt;
  __device__ void early() {}
  __device__ void issue(lds_t* dst) { issue_stage<FULL>(oa, ob, kt + 1, dst); }
};

// Main loop steps are instantiated by whether they load a next stage (PRE)
// and whether that stage needs bounds checks (!FULL), so the steady-state
// body has no branches: the leading full stages run first, the checked tail
// after.
template <int TMX, bool PRE, bool FULL, int SS = 0, class OA, class OB>
__device__ __forceinline__ void kstep(OA& oa, OB& ob, int kt, lds_t* base, int& slot,
                                      f32x16_t (&acc)[TMX][TN]) {
  SelfIssue<FULL, OA, OB> is{oa, ob, kt};
  kstep_core<TMX, PRE, SS, -1, OA, OB>(is, base, slot, acc);
  if constexpr (PRE) {
    oa.advance();
    ob.advance();
  }
}

// TMX: 32-row MFMA tiles per wave along M (a wave covers 32 TMX rows; the
// A operand holds WM * 32 TMX rows).
template <int TMX, class OA, class OB>
__device__ __forceinline__ void mainloop(OA& oa, OB& ob, int nk, char* smem, f32x16_t (&acc)[TMX][TN]) {
#pragma unroll
  for (int i = 0; i < TMX; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  lds_t* const base = (lds_t*)smem;
  // stages [0, nf) need no bounds checks
  const int nfa = oa.nfull(nk), nfb = ob.nfull(nk);
  const int nf = nfa < nfb ? nfa : nfb;
  if constexpr (OA::GATHERED || OB::GATHERED) {
    // the first stage of a gathered operand needs its row indices: wait for
    // them once, while nothing else is in flight (the compiler's own waits
    // would also cover each direct load issued in between), then issue that
    // operand first
    wait_vmcnt<0>();
    if constexpr (OB::GATHERED) {
      if (nf > 0) ob.template issue<0, OB::NI, true>(0, base + OA::BYTES);
      else ob.template issue<0, OB::NI, false>(0, base + OA::BYTES);
    }
    if (nf > 0) oa.template issue<0, OA::NI, true>(0, base);
    else oa.template issue<0, OA::NI, false>(0, base);
    if constexpr (!OB::GATHERED) {
      if (nf > 0) ob.template issue<0, OB::NI, true>(0, base + OA::BYTES);
      else ob.template issue<0, OB::NI, false>(0, base + OA::BYTES);
    }
  } else {
    if (nf > 0) issue_stage<true>(oa, ob, 0, base);
    else issue_stage<false>(oa, ob, 0, base);
  }
  oa.advance();
  ob.advance();
  int slot = 0, kt = 0;
  for (; kt + 1 < nf; ++kt) kstep<TMX, true, true>(oa, ob, kt, base, slot, acc);
  for (; kt + 1 < nk; ++kt) kstep<TMX, true, false>(oa, ob, kt, base, slot, acc);
  kstep<TMX, false, false>(oa, ob, kt, base, slot, acc);
}

// ---------------------------------------------------------------------------
// Five-slot ring for the forward GEMMs: five 32 KB slots of half stages, the
// weight slice (B) two K steps ahead and the token rows (A) one.  B_k sits
// in slot 2k mod 5 and A_k in slot 2k+1 mod 5; step k computes on slots
// s = 2k mod 5 and s+1, and issues A_{k+1} into slot s+3 (sub-step 0), then
// B_{k+2} into slot s+4 (sub-step 1); both slots held step k-1's operands,
// free after this step's barrier.  Against the two-stage ring this keeps
// half a stage more in flight in the same 160 KB, with one barrier per step.
// Step k waits until only B_{k+1}'s loads are outstanding (loads complete
// in issue order, and A_k left before them): A_k and B_k have landed.
// CHK: the steady-state stages need bounds checks (K is not a multiple of
// the step, or the tile's weight columns run past N).
// ---------------------------------------------------------------------------
constexpr int kSlot5 = 32 * 1024;
__device__ __forceinline__ int mod5(int v) { return v >= 5 ? v - 5 : v; }

template <int TMX, bool PRE_A, bool PRE_B, bool FULL, class OA, class OB>
__device__ __forceinline__ void kstep5_body(OA& oa, OB& ob, int k, const lds_t* __restrict__ As,
                                            const lds_t* __restrict__ Bs, lds_t* __restrict__ da,
                                            lds_t* __restrict__ db, f32x16_t (&acc)[TMX][TN]) {
  static_assert(OA::BYTES <= kSlot5 && OB::BYTES <= kSlot5, "five-slot ring operands");
  constexpr int NKK = BK / 16;
  const int wm = wave_m(), wn = wave_n();
  bf16x8_t a[2][TMX], b[2][TN];
#pragma unroll
  for (int i = 0; i < TMX; ++i) a[0][i] = OA::frag(As, wm * (TMX * 32) + i * 32, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) b[0][j] = OB::frag(Bs, wn * (TBN / WN) + j * 32, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int cur = kk & 1;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (kk + 1 < NKK) {
#pragma unroll
      for (int i = 0; i < TMX; ++i) a[cur ^ 1][i] = OA::frag(As, wm * (TMX * 32) + i * 32, kk + 1);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[cur ^ 1][j] = OB::frag(Bs, wn * (TBN / WN) + j * 32, kk + 1);
    }
    // A's loads in sub-step 0, B's in sub-step 1: the sub-step boundary
    // (sched_barrier) keeps them in that order, which the next step's
    // partial wait relies on (the __restrict__ slots would otherwise let
    // the compiler issue them in either order)
    if constexpr (PRE_A) {
      if (kk == 0) {
        oa.template issue<0, OA::NI, FULL>(k + 1, da);
        oa.advance();
      }
    }
    if constexpr (PRE_B) {
      if (kk == 1) {
        ob.template issue<0, OB::NI, FULL>(k + 2, db);
        ob.advance();
      }
    }
#pragma unroll
    for (int i = 0; i < TMX; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[cur][j], a[cur][i], acc[i][j], 0, 0, 0);
    // (a transposed fragment takes two reads)
    const int NR = kk + 1 < NKK ? TMX * (OA::TR ? 2 : 1) + TN * (OB::TR ? 2 : 1) : 0;
    const int NG = kk == 0 ? (PRE_A ? OA::NI : 0) : kk == 1 ? (PRE_B ? OB::NI : 0) : 0;
#pragma unroll
    for (int q = 0; q < TMX * TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
      if (q * 2 + 1 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
      else if (q * 2 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < NG) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// (The slots reach the body as __restrict__ parameters, as in kstep_body.)
template <int TMX, bool WAIT_B, bool PRE_A, bool PRE_B, bool FULL, class OA, class OB>
__device__ __forceinline__ void kstep5(OA& oa, OB& ob, int k, lds_t* base, int& s, f32x16_t (&acc)[TMX][TN]) {
  if constexpr (WAIT_B) wait_vmcnt<OB::NI>();
  else wait_vmcnt<0>();
  barrier_lds();
  // A_k in slot s + 1, B_k in slot s; A_{k+1} into s + 3, B_{k+2} into s + 4
  kstep5_body<TMX, PRE_A, PRE_B, FULL>(oa, ob, k, base + mod5(s + 1) * kSlot5, base + s * kSlot5,
                                       base + mod5(s + 3) * kSlot5, base + mod5(s + 4) * kSlot5, acc);
  s = mod5(s + 2);
}

template <int TMX, bool CHK, class OA, class OB>
__device__ __forceinline__ void mainloop5(OA& oa, OB& ob, int nk, char* smem, f32x16_t (&acc)[TMX][TN]) {
#pragma unroll
  for (int i = 0; i < TMX; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  lds_t* const base = (lds_t*)smem;
  // prologue: B_0 (slot 0), A_0 (slot 1), B_1 (slot 2); with !CHK every
  // stage is whole
  ob.template issue<0, OB::NI, !CHK>(0, base);
  ob.advance();
  oa.template issue<0, OA::NI, !CHK>(0, base + kSlot5);
  oa.advance();
  if (nk > 1) {
    ob.template issue<0, OB::NI, !CHK>(1, base + 2 * kSlot5);
    ob.advance();
  }
  int s = 0, k = 0;
  for (; k + 2 < nk; ++k) kstep5<TMX, true, true, true, !CHK>(oa, ob, k, base, s, acc);
  if (k + 1 < nk) {
    kstep5<TMX, true, true, false, !CHK>(oa, ob, k, base, s, acc);
    ++k;
  }
  kstep5<TMX, false, false, false, false>(oa, ob, k, base, s, acc);
}

// Accumulator layout.  The MFMAs take the B fragment as their first
// operand, so tile (i, j) holds the transpose of the usual output: lane l
// has row i * 32 + (l & 31) of the wave tile, and register r its column
// j * 32 + 8 (r / 4) + 4 (l / 32) + r % 4.  Each group of four registers is
// four consecutive columns of one row: one 8-byte bf16 write.
__device__ __forceinline__ int acc_row(int i, int lane) { return i * 32 + (lane & 31); }
__device__ __forceinline__ int acc_col(int j, int g, int lane) { return j * 32 + 8 * g + 4 * (lane >> 5); }

// ---------------------------------------------------------------------------
// Epilogue staging: accumulators -> bf16 tile in LDS (row stride S bytes) ->
// 16-byte coalesced rows in global memory.
// ---------------------------------------------------------------------------
template <int COLS>
constexpr int ep_stride() { return COLS * 2 + 16; }

// Writes the wave's MFMA tiles i in [0, NI), j in [0, NJ), value v(i, j, r),
// at tile rows row0.. and columns col0.., four columns (8 bytes) a write.
template <int NI, int NJ, int S, class V>
__device__ __forceinline__ void stage_quads(lds_t* t, int row0, int col0, V v, int tid = threadIdx.x) {
  const int lane = tid & 63;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t w = {pack_bf16x2(v(i, j, 4 * g), v(i, j, 4 * g + 1)),
                           pack_bf16x2(v(i, j, 4 * g + 2), v(i, j, 4 * g + 3))};
        const int row = row0 + acc_row(i, lane), col = col0 + acc_col(j, g, lane);
        *(__attribute__((address_space(3))) u32x2_t*)(t + row * S + col * 2) = w;
      }
}

struct RowId {
  __device__ int operator()(int r) const { return r; }
};

// Copies the staged ROWS x COLS tile to C (leading dimension ldc elements):
// staged row s is row map(s) of C; rows >= row_lim and columns >= col_lim
// are skipped.
template <int ROWS, int COLS, int S, class M = RowId>
__device__ __forceinline__ void lds_to_global(const lds_t* t, bf16_t* C, int64_t ldc, int row_lim,
                                              int col_lim, M map = M(), int tid = threadIdx.x) {
  constexpr int CPR = COLS / 8;  // 16-byte chunks per row
  constexpr int NQ = ROWS * CPR / NTHR;
  static_assert(ROWS * CPR % NTHR == 0, "whole chunks per thread");
  // all of the thread's LDS reads first, so the stores leave back to back
  u32x4_t v[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = tid + i * NTHR;
    v[i] = *(const __attribute__((address_space(3))) u32x4_t*)(t + (q / CPR) * S + (q % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = tid + i * NTHR;
    const int row = map(q / CPR), c8 = q % CPR;
    if (row < row_lim && c8 * 8 < col_lim)  // streamed out: no L2 line kept for the output
      __builtin_nontemporal_store(v[i], (u32x4_t*)(C + (int64_t)row * ldc + c8 * 8));
  }
}

// ===========================================================================
// Ragged-M GEMMs: rows are an expert's segment of the expert-sorted rows.
// ===========================================================================
enum Epi { EPI_STORE = 0, EPI_GATEUP = 1 };
enum BLay { B_MK = 0, B_MK_GATEUP = 1, B_KM = 2 };

struct RowsArgs {
  // A(row, k) = A[arow(row) * lda + k], arow = a_src ? a_src[row] / a_div : row
  const bf16_t* A;
  int64_t lda;
  const int32_t* a_src;
  int a_div;
  // B_MK:        B(n, k) = Be[n * ldb + k]
  // B_MK_GATEUP: B(n, k) = Be[wrow(n) * ldb + k]; 32-row blocks alternate
  //              gate rows (even block) and up rows (odd block)
  // B_KM:        B(n, k) = Be[k * ldb + n]
  const bf16_t* B;
  int64_t b_estride, ldb;
  int N, K, n_tiles;  // N: output columns (gate/up: gate columns I)
  int row_major;      // tile order within an expert (rows_tile_order)
  const int32_t* offsets;
  const int32_t* tile_off;
  const int4* tiles;  // row-tile descriptors {expert, first row, segment end, expert's first tile}
  int E;
  // EPI_STORE: C [R, ldc]
  bf16_t* C;
  int64_t ldc;
  // EPI_GATEUP: H [R,2I] (optional), Aw [R,I] = w_row * silu(g) * u (g, u
  // clamped at lim: +inf for the plain SwiGLU)
  bf16_t* H;
  bf16_t* Aout;
  int I;
  float lim;
  const float* topk_w;
  const int32_t* src_of;
};

// Rows of a row tile that instruction i of OpMK<ROWS> loads: through a_src
// (the gather) or plain; rows past the segment repeat the tile's first row
// (computed, never stored).
template <int ROWS>
__device__ __forceinline__ void fetch_arow(const RowsArgs& p, int m0, int seg1, int (&arow)[OpMK<ROWS>::NI]) {
#pragma unroll
  for (int i = 0; i < OpMK<ROWS>::NI; ++i) {
    int r = m0 + OpMK<ROWS>::lane_row(i);
    if (r >= seg1) r = m0;
    arow[i] = p.a_src ? p.a_src[r] : r;
  }
}

template <int ROWS>
__device__ __forceinline__ void init_a(const RowsArgs& p, OpMK<ROWS>& oa, const int (&arow)[OpMK<ROWS>::NI]) {
  oa.init([&](int i, int) {
    const int64_t ar = p.a_src ? (int64_t)(arow[i] / p.a_div) : (int64_t)arow[i];
    return p.A + ar * p.lda;
  }, p.K);
}

// The B operand of expert e's N tile nt.
template <int BL> struct BOperand { using type = OpMK<TBN>; };
template <> struct BOperand<B_KM> { using type = OpKM<TBN>; };

template <int BL>
__device__ __forceinline__ void init_b(const RowsArgs& p, typename BOperand<BL>::type& ob, int e, int nt) {
  const bf16_t* Be = p.B + (int64_t)e * p.b_estride;
  if constexpr (BL == B_KM) {
    ob.init(Be, p.ldb, nt * TBN, p.N, p.K);
  } else {
    ob.init([&](int, int n) {
      int wrow;
      if constexpr (BL == B_MK_GATEUP) {
        const int blk = n >> 5;
        int gc = nt * (TBN / 2) + (blk >> 1) * 32 + (n & 31);
        if (gc >= p.I) gc = 0;
        wrow = (blk & 1) ? p.I + gc : gc;
      } else {
        wrow = nt * TBN + n;
        if (wrow >= p.N) wrow = 0;
      }
      return Be + (int64_t)wrow * p.ldb;
    }, p.K);
  }
}

// 1 + the flat (token, slot) entry of tile row threadIdx.x, 0 for none: the
// gate/up epilogue's row weight is topk_w at that entry.
template <int ROWS>
__device__ __forceinline__ int fetch_wsrc(const RowsArgs& p, int m0, int seg1) {
  return threadIdx.x < ROWS && m0 + (int)threadIdx.x < seg1 ? p.src_of[m0 + threadIdx.x] + 1 : 0;
}

// One row tile: ROWS = 256, or 128 / 64 for a segment's last tile when it
// holds at most that many rows (the waves then take 64 / 32 rows each: a
// half / a quarter of the MFMA work and of the A operand, where a full tile
// would spend most of it on rows past the segment).
template <int EPI, int BL, int ROWS>
__device__ __forceinline__ void rows_tile(const RowsArgs& p, char* smem, int nt, int e, int m0, int seg1) {
  constexpr int TMX = ROWS / WM / 32;
  const int lane = threadIdx.x & 63;
  const int wm = wave_m(), wn = wave_n();

  // The loads whose results the prologue needs leave together: the gate/up
  // epilogue's row weights (flat entry first; the main loop hides the
  // second, dependent load) and the gathered A rows.  Address math between
  // loads made the compiler wait for each before issuing the next.
  int wsrc = 0;
  if constexpr (EPI == EPI_GATEUP) wsrc = fetch_wsrc<ROWS>(p, m0, seg1);
  int arow[OpMK<ROWS>::NI];
  fetch_arow<ROWS>(p, m0, seg1, arow);
  float wrow = 0.0f;
  if constexpr (EPI == EPI_GATEUP) {
    if (wsrc) wrow = p.topk_w[wsrc - 1];
  }
  OpMK<ROWS> oa;
  init_a<ROWS>(p, oa, arow);
  typename BOperand<BL>::type ob;
  init_b<BL>(p, ob, e, nt);
  f32x16_t acc[TMX][TN];
  const int nk = (int)cdiv(p.K, BK);
  if constexpr (BL == B_KM) {
    // the data gradients stay on the two-stage ring: on the five-slot ring
    // they ran 1-5% slower (q235b: both; q30b: the down dgrad)
    mainloop<TMX>(oa, ob, nk, smem, acc);
  } else if (oa.nfull(nk) == nk && ob.nfull(nk) == nk) {
    mainloop5<TMX, false>(oa, ob, nk, smem, acc);
  } else {
    mainloop5<TMX, true>(oa, ob, nk, smem, acc);
  }

  // ------------------------------------------------------------- epilogues
  // The LDS ring is free once every wave has left the main loop.
  barrier_lds();
  lds_t* const lds = (lds_t*)smem;
  const int rows_valid = seg1 - m0;  // rows of this tile inside the segment (may exceed ROWS)
  const int r0w = wm * (ROWS / WM);  // first tile row of this wave
  if constexpr (EPI == EPI_STORE) {
    constexpr int S = ep_stride<TBN>();
    stage_quads<TMX, TN, S>(lds, r0w, wn * (TBN / WN), [&](int i, int j, int r) { return acc[i][j][r]; });
    barrier_lds();
    lds_to_global<ROWS, TBN, S>(lds, p.C + (int64_t)m0 * p.ldc + nt * TBN, p.ldc, rows_valid,
                                p.N - nt * TBN);
  } else if constexpr (EPI == EPI_GATEUP) {
    // acc[i][0] = gate, acc[i][1] = up, register by register for the same
    // gate column wn * 32 + acc_col(0, r / 4, lane) + r % 4 (128 gate columns
    // per tile)
    constexpr int S = ep_stride<TBN / 2>();
    constexpr int TB = ROWS * S;  // bytes of one staged ROWS x 128 tile
    lds_f32_t* wl = (lds_f32_t*)(lds + 2 * TB);
    if (threadIdx.x < ROWS) wl[threadIdx.x] = wrow;
    barrier_lds();
    const int c0w = wn * 32;
    stage_quads<TMX, 1, S>(lds, r0w, c0w, [&](int i, int, int r) {
      const float g = clamp_gate(acc[i][0][r], p.lim), u = clamp_up(acc[i][1][r], p.lim);
      return wl[r0w + acc_row(i, lane)] * (g * sigmoidf_(g) * u);
    });
    if (p.H) stage_quads<TMX, 1, S>(lds + TB, r0w, c0w, [&](int i, int, int r) { return acc[i][0][r]; });
    barrier_lds();
    const int gc0 = nt * (TBN / 2);
    lds_to_global<ROWS, TBN / 2, S>(lds, p.Aout + (int64_t)m0 * p.I + gc0, p.I, rows_valid, p.I - gc0);
    if (p.H) {
      bf16_t* H0 = p.H + (int64_t)m0 * 2 * p.I + gc0;
      lds_to_global<ROWS, TBN / 2, S>(lds + TB, H0, 2 * p.I, rows_valid, p.I - gc0);
      barrier_lds();
      stage_quads<TMX, 1, S>(lds, r0w, c0w, [&](int i, int, int r) { return acc[i][1][r]; });
      barrier_lds();
      lds_to_global<ROWS, TBN / 2, S>(lds, H0 + p.I, 2 * p.I, rows_valid, p.I - gc0);
    }
  }
}

struct RowTile {
  int e, nt, m0, seg1;
};

// Logical tile L: an expert's (row tile, N tile) pairs are a contiguous
// range of L, taken N-tile-major (work-groups that run close together share
// a weight tile through L2) or, with row_major, row-tile-major (they share
// token rows); the descriptor of L's row-tile-major row tile lies in the
// same expert and gives the range.
__device__ __forceinline__ RowTile decode_tile(const RowsArgs& p, int L) {
  const int T = L / p.n_tiles;
  // {expert, first row, segment end, expert's first tile}, read through the
  // constant address space: a scalar load, so that in the persistent loop
  // waiting for it does not wait for the direct loads in flight
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  const i32x4_t d0 = ((const __attribute__((address_space(4))) i32x4_t*)p.tiles)[T];
  const int first = d0.w;
  const int seg0 = d0.y - (T - first) * TBM;
  const int nrt = (d0.z - seg0 + TBM - 1) / TBM;
  const int j = L - first * p.n_tiles;
  RowTile t;
  t.e = d0.x;
  t.seg1 = d0.z;
  const int rt = p.row_major ? j / p.n_tiles : j % nrt;
  t.nt = p.row_major ? j - rt * p.n_tiles : j / nrt;
  t.m0 = seg0 + rt * TBM;
  return t;
}

// TAG only tells launch sites with the same epilogue and B layout apart in
// profiles.
template <int EPI, int BL, int TAG>
__global__ __launch_bounds__(NTHR, 1) void rows_gemm_kernel(RowsArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int L = xcd_tile(blockIdx.x, p.tile_off[p.E] * p.n_tiles);
  if (L < 0) return;
  const RowTile t = decode_tile(p, L);
  const int e = t.e, nt = t.nt, m0 = t.m0, seg1 = t.seg1;
  const int rows = seg1 - m0;
  if (rows <= TBM / 4) rows_tile<EPI, BL, TBM / 4>(p, smem, nt, e, m0, seg1);
  else if (rows <= TBM / 2) rows_tile<EPI, BL, TBM / 2>(p, smem, nt, e, m0, seg1);
  else rows_tile<EPI, BL, TBM>(p, smem, nt, e, m0, seg1);
}

// ===========================================================================
// Persistent ragged-M GEMM: one work-group per CU walks its XCD's tiles
// (the same contiguous eighth of the launch's tiles as above, dealt
// round-robin to the XCD's work-groups), all at full height.  The first
// stage of the next tile - its gathered token rows and its weight slice -
// is issued in the current tile's last K step, so it loads while that
// step's MFMAs run and while the epilogue stages and stores; the next tile
// starts on a landed stage.  This is the one-GPU form of a persistent
// kernel that moves the next token group while it computes on the current
// one ("Prime Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster",
// section "One kernel overlaps the pipeline").
//
// LDS: slot 0 at [0, 64K), slot 1 at [96K, 160K).  The 32 KB between them
// joins the slot the last step read to give the epilogue a 96 KB staging
// area that the next tile's first stage, in the other slot, never touches.
// ===========================================================================
constexpr int kPSlot = 96 * 1024;
constexpr size_t kPSmem = (size_t)kPSlot + (size_t)(TBM + TBN) * BK * 2;
static_assert(kPSmem <= 160 * 1024, "LDS");

// Issues the next tile's first stage (if there is one: `more`) in the
// current tile's last K step: its row indices (and the gate/up epilogue's
// row-weight entries) load right after the step's barrier, its direct loads
// leave in the last sub-step, bounds-checked (once per tile: one form of the
// step serves every tile).  oa / ob become the next tile's operands,
// advanced past that stage.
template <int EPI, int BL>
struct NextIssue {
  const RowsArgs& p;
  const RowTile& t;
  bool more;
  OpMK<TBM>& oa;
  typename BOperand<BL>::type& ob;
  float& wrow;
  int arow[OpMK<TBM>::NI];
  int wsrc;
  __device__ void early() {
    if (!more) return;
    fetch_arow<TBM>(p, t.m0, t.seg1, arow);
    if constexpr (EPI == EPI_GATEUP) wsrc = fetch_wsrc<TBM>(p, t.m0, t.seg1);
  }
  __device__ void issue(lds_t* dst) {
    if (!more) return;
    init_a<TBM>(p, oa, arow);
    init_b<BL>(p, ob, t.e, t.nt);
    issue_stage<false>(oa, ob, 0, dst);
    oa.advance();
    ob.advance();
    if constexpr (EPI == EPI_GATEUP) wrow = wsrc ? p.topk_w[wsrc - 1] : 0.0f;
  }
};

// threadIdx.x, taken afresh: values derived from it in a tile's epilogue
// are not hoisted out of the persistent loop (where they would stay live
// through the main loop).
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Plain store of a full 256 x 256 tile to C0 (leading dimension ldc; rows
// >= row_lim and columns >= col_lim skipped), staged inside the 96 KB area
// beside slot `last ^ 1` (which holds the next tile's first stage) in two
// rounds of 128 rows: round h holds the waves' MFMA row tiles 2h and 2h + 1,
// so staged row s is tile row (s / 64) * 128 + 64 h + s % 64.
__device__ __forceinline__ void persist_store(lds_t* base, int last, f32x16_t (&acc)[TM][TN], bf16_t* C0,
                                              int64_t ldc, int row_lim, int col_lim) {
  const int tid = fresh_tid();
  const int wm = (tid >> 6) / WN, wn = (tid >> 6) % WN;
  constexpr int S = ep_stride<TBN>();
  static_assert(128 * S <= kPSlot && 64 * 1024 + 128 * S <= (int)kPSmem, "staging area beside either slot");
  lds_t* const stg = base + (last ? 64 * 1024 : 0);
  barrier_lds();  // every wave is done with the last step's slot
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h) barrier_lds();
    stage_quads<2, TN, S>(stg, wm * 64, wn * (TBN / WN), [&](int i, int j, int r) { return acc[2 * h + i][j][r]; }, tid);
    barrier_lds();
    lds_to_global<128, TBN, S>(stg, C0, ldc, row_lim, col_lim,
                               [h](int s) { return (s >> 6) * 128 + h * 64 + (s & 63); }, tid);
  }
}

// Epilogue of a full-height tile, staged inside the 96 KB area beside slot
// `last ^ 1` (which holds the next tile's first stage).
template <int EPI>
__device__ __forceinline__ void persist_epilogue(const RowsArgs& p, const RowTile& t, lds_t* base, int last,
                                                 f32x16_t (&acc)[TM][TN], float wrow) {
  const int tid = fresh_tid(), lane = tid & 63;
  const int wm = (tid >> 6) / WN, wn = (tid >> 6) % WN;
  const int rows_valid = t.seg1 - t.m0;
  if constexpr (EPI == EPI_STORE) {
    persist_store(base, last, acc, p.C + (int64_t)t.m0 * p.ldc + t.nt * TBN, p.ldc, rows_valid, p.N - t.nt * TBN);
  } else {
    // three rounds of 256 x 128: Aw, then H's gate and up columns; the row
    // weights sit in the 32 KB gap, clear of both the staged tile and the
    // slots, so they are written before the first barrier
    constexpr int S = ep_stride<TBN / 2>();
    constexpr int TB = TBM * S;
    static_assert(TB + 1024 <= kPSlot && 65 * 1024 + TB <= (int)kPSmem, "staging area beside either slot");
    lds_t* const stg = base + (last ? 65 * 1024 : 0);
    lds_f32_t* const wl = (lds_f32_t*)(base + (last ? 64 * 1024 : TB));
    if (tid < TBM) wl[tid] = wrow;
    barrier_lds();
    const int r0w = wm * (TBM / WM), c0w = wn * 32;
    const int gc0 = t.nt * (TBN / 2);
    stage_quads<TM, 1, S>(stg, r0w, c0w, [&](int i, int, int r) {
      const float g = clamp_gate(acc[i][0][r], p.lim), u = clamp_up(acc[i][1][r], p.lim);
      return wl[r0w + acc_row(i, lane)] * (g * sigmoidf_(g) * u);
    }, tid);
    barrier_lds();
    lds_to_global<TBM, TBN / 2, S>(stg, p.Aout + (int64_t)t.m0 * p.I + gc0, p.I, rows_valid, p.I - gc0, RowId(), tid);
    if (p.H) {
      bf16_t* H0 = p.H + (int64_t)t.m0 * 2 * p.I + gc0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        barrier_lds();
        stage_quads<TM, 1, S>(stg, r0w, c0w, [&](int i, int, int r) { return acc[i][h][r]; }, tid);
        barrier_lds();
        lds_to_global<TBM, TBN / 2, S>(stg, H0 + h * p.I, 2 * p.I, rows_valid, p.I - gc0, RowId(), tid);
      }
    }
  }
}

template <int EPI, int BL, int TAG>
__global__ __launch_bounds__(NTHR, 1) void rows_persist_kernel(RowsArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  using OB = typename BOperand<BL>::type;
  const int real = p.tile_off[p.E] * p.n_tiles;
  const int per = (real + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int P = (int)(gridDim.x >> 3);  // work-groups per XCD
  const int end = min(xcd * per + per, real);
  int L = xcd * per + (int)(blockIdx.x >> 3);
  if (L >= end) return;
  lds_t* const base = (lds_t*)smem;
  const int nk = (int)cdiv(p.K, BK);  // >= 1 (the host launches K >= 1 only)
  RowTile t = decode_tile(p, L);
  OpMK<TBM> oa;
  OB ob;
  float wrow = 0.0f;
  {  // the first tile's first stage
    int wsrc = 0;
    if constexpr (EPI == EPI_GATEUP) wsrc = fetch_wsrc<TBM>(p, t.m0, t.seg1);
    int arow[OpMK<TBM>::NI];
    fetch_arow<TBM>(p, t.m0, t.seg1, arow);
    if constexpr (EPI == EPI_GATEUP) {
      if (wsrc) wrow = p.topk_w[wsrc - 1];
    }
    init_a<TBM>(p, oa, arow);
    init_b<BL>(p, ob, t.e, t.nt);
    issue_stage<false>(oa, ob, 0, base);
    oa.advance();
    ob.advance();
  }
  int slot = 0;
  for (;;) {
    const int Ln = L + P;
    const bool more = Ln < end;
    const RowTile tn = decode_tile(p, more ? Ln : L);
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int nfa = oa.nfull(nk), nfb = ob.nfull(nk);
    const int nf = nfa < nfb ? nfa : nfb;
    int kt = 0;
    for (; kt + 1 < nf; ++kt) kstep<TM, true, true, kPSlot>(oa, ob, kt, base, slot, acc);
    for (; kt + 1 < nk; ++kt) kstep<TM, true, false, kPSlot>(oa, ob, kt, base, slot, acc);
    const int last = slot;
    float wnext = 0.0f;
    {
      NextIssue<EPI, BL> is{p, tn, more, oa, ob, wnext};
      kstep_core<TM, true, kPSlot, BK / 16 - 1, OpMK<TBM>, OB>(is, base, slot, acc);
    }
    persist_epilogue<EPI>(p, t, base, last, acc, wrow);
    if (!more) break;
    L = Ln;
    t = tn;
    wrow = wnext;
  }
}

// ===========================================================================
// Weight gradients: dW[e][m, n] = sum over the expert's rows r of
// A[seg0 + r][m] * B[seg0 + r][n]; both operands are row-major [R, *] with
// rows in expert order (contiguous per expert).
// ===========================================================================
struct WgradArgs {
  // A(m, r) = A[arow(r) * lda + m], B(n, r) = B[brow(r) * ldb + n]; the
  // gathered side (TAG 0: A, TAG 1: B) reads row tok[r], the other row r
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  const int32_t* tok;  // [R] token of each expert-sorted row
  int M, N, m_tiles, n_tiles, E;
  const int32_t* offsets;
  const int32_t* xorder;  // expert of each (slot, XCD): see the schedule
  bf16_t* C;  // dW[e] = C + e * c_estride, row-major [M, N]
  int64_t c_estride;
};

// All tiles of an expert run on one XCD (work-groups go to XCD bid % 8), so
// its rows are fetched into one L2; the schedule deals the experts to the
// XCDs so that their rows balance (xorder).
// TAG 0: the down wgrad (A = dout gathered by token), 1: the gate/up wgrad
// (B = x gathered by token).
template <int TAG>
__global__ __launch_bounds__(NTHR, 1) void wgrad_kernel(WgradArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int per = p.m_tiles * p.n_tiles;
  const int slot = (blockIdx.x >> 3) / per;  // the work-group runs on XCD blockIdx.x % 8
  if (slot >= (p.E + 7) / 8) return;
  const int e = p.xorder[slot * 8 + (blockIdx.x & 7)];
  if (e < 0) return;
  const int rem = (blockIdx.x >> 3) % per;
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int seg0 = p.offsets[e];
  const int len = p.offsets[e + 1] - seg0;
  OpKMg<TBM, TAG == 0> oa;
  OpKMg<TBN, TAG == 1> ob;
  oa.init(p.A, p.lda, p.tok, seg0, mt * TBM, p.M, len);
  ob.init(p.B, p.ldb, p.tok, seg0, nt * TBN, p.N, len);
  f32x16_t acc[TM][TN];
  mainloop<TM>(oa, ob, (int)cdiv(len, BK), smem, acc);
  barrier_lds();
  lds_t* const lds = (lds_t*)smem;
  constexpr int S = ep_stride<TBN>();
  stage_quads<TM, TN, S>(lds, wave_m() * (TBM / WM), wave_n() * (TBN / WN),
                         [&](int i, int j, int r) { return acc[i][j][r]; });
  barrier_lds();
  lds_to_global<TBM, TBN, S>(lds, p.C + (int64_t)e * p.c_estride + (int64_t)mt * TBM * p.N + nt * TBN,
                             p.N, p.M - mt * TBM, p.N - nt * TBN);
}

// ===========================================================================
// Persistent weight gradients: one work-group per CU walks its XCD's tiles
// (the tiles wgrad_kernel deals to that XCD, in the same order) with stride
// the XCD's work-group count, and issues the next tile's first stage in the
// current tile's last K step, so that it loads during that step's MFMAs and
// the epilogue (the LDS plan of the persistent row GEMMs: slots at 0 and
// 96 KB, the epilogue staged beside the slot being filled).  Tiles of
// experts with no rows are written as zeros directly, outside the pipeline.
// ===========================================================================
struct WTile {
  int e, mt, nt, seg0, len;
};

struct WgradWalk {
  const WgradArgs& p;
  int xcd, per, total, stride;

  // The schedule is read through the constant address space, so these
  // uniform loads are scalar: waiting for them (lgkmcnt) does not wait for
  // the direct loads in flight, as a vector load's vmcnt would.
  __device__ WTile at(int j) const {
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    WTile t;
    const int s = j / per, rem = j - s * per;
    t.e = ((cptr)p.xorder)[s * 8 + xcd];
    t.mt = rem / p.n_tiles;
    t.nt = rem - t.mt * p.n_tiles;
    t.seg0 = t.e >= 0 ? ((cptr)p.offsets)[t.e] : 0;
    t.len = t.e >= 0 ? ((cptr)p.offsets)[t.e + 1] - t.seg0 : 0;
    return t;
  }
  // zeros for the tile of an expert with no rows
  __device__ void zero_tile(const WTile& t) const {
    constexpr int CPR = TBN / 8;
    bf16_t* const C0 = p.C + (int64_t)t.e * p.c_estride + (int64_t)t.mt * TBM * p.N + t.nt * TBN;
    const int row_lim = p.M - t.mt * TBM, col_lim = p.N - t.nt * TBN;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int q = (int)threadIdx.x; q < TBM * CPR; q += NTHR) {
      const int row = q / CPR, c8 = q % CPR;
      if (row < row_lim && c8 * 8 < col_lim)
        __builtin_nontemporal_store(z, (u32x4_t*)(C0 + (int64_t)row * p.N + c8 * 8));
    }
  }
  // the first of this work-group's tiles at or after j whose expert has
  // rows (total if none), zeroing the empty experts' tiles passed on the way
  __device__ int next(int j, WTile& t) const {
    for (; j < total; j += stride) {
      t = at(j);
      if (t.e < 0) continue;
      if (t.len > 0) return j;
      zero_tile(t);
    }
    return total;
  }
};

// Issues the next tile's first stage in the current tile's last K step: its
// row indices load right after the step's barrier, its direct loads leave in
// the last sub-step (bounds-checked); oa / ob become the next tile's
// operands, advanced past that stage.
template <int TAG>
struct WNextIssue {
  const WgradArgs& p;
  const WTile& t;
  bool more;
  OpKMg<TBM, TAG == 0>& oa;
  OpKMg<TBN, TAG == 1>& ob;
  __device__ void early() {
    if (!more) return;
    oa.init(p.A, p.lda, p.tok, t.seg0, t.mt * TBM, p.M, t.len);
    ob.init(p.B, p.ldb, p.tok, t.seg0, t.nt * TBN, p.N, t.len);
  }
  __device__ void issue(lds_t* dst) {
    if (!more) return;
    issue_stage<false>(oa, ob, 0, dst);
    oa.advance();
    ob.advance();
  }
};

template <int TAG>
__global__ __launch_bounds__(NTHR, 1) void wgrad_persist_kernel(WgradArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  using OA = OpKMg<TBM, TAG == 0>;
  using OB = OpKMg<TBN, TAG == 1>;
  const int per = p.m_tiles * p.n_tiles;
  const WgradWalk w{p, (int)(blockIdx.x & 7), per, (p.E + 7) / 8 * per, (int)(gridDim.x >> 3)};
  WTile t;
  int j = w.next((int)(blockIdx.x >> 3), t);
  if (j >= w.total) return;
  lds_t* const base = (lds_t*)smem;
  OA oa;
  OB ob;
  oa.init(p.A, p.lda, p.tok, t.seg0, t.mt * TBM, p.M, t.len);
  ob.init(p.B, p.ldb, p.tok, t.seg0, t.nt * TBN, p.N, t.len);
  wait_vmcnt<0>();  // the first stage's row indices
  issue_stage<false>(oa, ob, 0, base);
  oa.advance();
  ob.advance();
  int slot = 0;
  for (;;) {
    WTile tn;
    const int jn = w.next(j + w.stride, tn);
    const bool more = jn < w.total;
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
    const int nk = (int)cdiv(t.len, BK);  // >= 1: empty experts never get here
    const int nfa = oa.nfull(nk), nfb = ob.nfull(nk);
    const int nf = nfa < nfb ? nfa : nfb;
    int kt = 0;
    for (; kt + 1 < nf; ++kt) kstep<TM, true, true, kPSlot>(oa, ob, kt, base, slot, acc);
    for (; kt + 1 < nk; ++kt) kstep<TM, true, false, kPSlot>(oa, ob, kt, base, slot, acc);
    const int last = slot;
    {
      WNextIssue<TAG> is{p, tn, more, oa, ob};
      kstep_core<TM, true, kPSlot, BK / 16 - 1, OA, OB>(is, base, slot, acc);
    }
    persist_store(base, last, acc,
                  p.C + (int64_t)t.e * p.c_estride + (int64_t)t.mt * TBM * p.N + t.nt * TBN, p.N,
                  p.M - t.mt * TBM, p.N - t.nt * TBN);
    if (!more) break;
    j = jn;
    t = tn;
  }
}

// Dynamic LDS: the operand ring, or the largest epilogue staging area.
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t kRingBytes = (size_t)NSTAGE * (TBM + TBN) * BK * 2;
constexpr size_t kStoreEpi = (size_t)TBM * ep_stride<TBN>();
constexpr size_t kGateupEpi = (size_t)2 * TBM * ep_stride<TBN / 2>() + TBM * 4;
constexpr size_t kSmem = cmax(cmax(kRingBytes, (size_t)5 * kSlot5), cmax(kStoreEpi, kGateupEpi));
static_assert(kSmem <= 160 * 1024, "LDS");

template <int EPI, int BL, int TAG = 0>
hipError_t launch_rows_tiles(const LaunchCtx& c, const char* name, RowsArgs p, int R) {
  {
    hipError_t e = allow_smem_once<rows_gemm_kernel<EPI, BL, TAG>>(kSmem);
    if (e != hipSuccess) return e;
  }
  // upper bound of the tile count (the kernel reads the exact one)
  const int64_t tiles = (int64_t)(R / TBM + p.E) * p.n_tiles;
  const unsigned nblocks = (unsigned)((tiles + 7) / 8 * 8);
  MOE_LAUNCH(c, name, (rows_gemm_kernel<EPI, BL, TAG>), dim3(nblocks), dim3(NTHR), kSmem, p);
  return hipSuccess;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The persistent form: one work-group per CU, at most as many per XCD as
// the XCD can have tiles.
template <int EPI, int BL, int TAG = 0>
hipError_t launch_rows_persist(const LaunchCtx& c, const char* name, RowsArgs p, int R) {
  {
    hipError_t e = allow_smem_once<rows_persist_kernel<EPI, BL, TAG>>(kPSmem);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = (int64_t)(R / TBM + p.E) * p.n_tiles;  // upper bound of the tile count
  const int64_t per_xcd = std::min<int64_t>(std::max(cu_count() / 8, 1), cdiv(tiles, 8));
  MOE_LAUNCH(c, name, (rows_persist_kernel<EPI, BL, TAG>), dim3((unsigned)(8 * per_xcd)), dim3(NTHR), kPSmem, p);
  return hipSuccess;
}

template <int TAG>
hipError_t launch_wgrad(const LaunchCtx& c, const char* name, const WgradArgs& p, int E, bool persistent) {
  const int64_t per_xcd_tiles = cdiv(E, 8) * p.m_tiles * p.n_tiles;
  if (persistent) {
    hipError_t e = allow_smem_once<wgrad_persist_kernel<TAG>>(kPSmem);
    if (e != hipSuccess) return e;
    const int64_t per_xcd = std::min<int64_t>(std::max(cu_count() / 8, 1), per_xcd_tiles);
    MOE_LAUNCH(c, name, wgrad_persist_kernel<TAG>, dim3((unsigned)(8 * per_xcd)), dim3(NTHR), kPSmem, p);
    return hipSuccess;
  }
  {
    hipError_t e = allow_smem_once<wgrad_kernel<TAG>>(kSmem);
    if (e != hipSuccess) return e;
  }
  const unsigned nblocks = (unsigned)(8 * per_xcd_tiles);
  MOE_LAUNCH(c, name, wgrad_kernel<TAG>, dim3(nblocks), dim3(NTHR), kSmem, p);
  return hipSuccess;
}

}  // namespace

// Row GEMMs: the persistent form on request (K >= 1 always holds here).
template <int EPI, int BL, int TAG = 0>
hipError_t launch_rows(const LaunchCtx& c, const char* name, const RowsArgs& p, int R, bool persistent) {
  if (persistent && p.K >= 1) return launch_rows_persist<EPI, BL, TAG>(c, name, p, R);
  return launch_rows_tiles<EPI, BL, TAG>(c, name, p, R);
}

int bf16_dw_blocks(int) { return 1; }

hipError_t bf16_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aw, void* Yw) {
  const int64_t I = a.I, d = a.d;
  {  // gate/up GEMM: token rows gathered from x; SwiGLU and top-k weight in the epilogue
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = (const bf16_t*)a.x; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, TBN / 2);
    p.row_major = rows_tile_order(a.T * d, a.E * 2 * I * d);
    p.H = (bf16_t*)H; p.Aout = (bf16_t*)Aw; p.I = a.I; p.lim = a.swiglu_lim;
    p.topk_w = a.topk_w; p.src_of = a.src_of;
    hipError_t err = launch_rows<EPI_GATEUP, B_MK_GATEUP>(c, "gemm_gateup_fwd", p, a.R, a.persistent);
    if (err != hipSuccess) return err;
  }
  if (!Yw) return hipSuccess;  // the gate/up half alone (recomputation)
  // down GEMM: Yw = Aw W_down[e]^T (rows already carry their top-k weight)
  RowsArgs q = {};
  q.offsets = a.offsets; q.tile_off = a.tile_off; q.tiles = a.tiles; q.E = a.E;
  q.A = (const bf16_t*)Aw; q.lda = I; q.a_src = nullptr; q.a_div = 1;
  q.B = (const bf16_t*)a.w_down; q.b_estride = d * I; q.ldb = I;
  q.N = a.d; q.K = a.I; q.n_tiles = (int)cdiv(a.d, TBN);
  q.row_major = rows_tile_order(a.R * I, a.E * d * I);
  q.C = (bf16_t*)Yw; q.ldc = d;
  return launch_rows<EPI_STORE, B_MK>(c, "gemm_down_fwd", q, a.R, a.persistent);
}

hipError_t bf16_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout,
                          const void* H, const void* Aw, void* dH, void* dXp, float* dwp,
                          void* dW_gu, void* dW_d) {
  const int64_t I = a.I, d = a.d;
  hipError_t err;
  {  // down dgrad: G = dout_t W_down[e] (into the dXp buffer, free until the
     // gate/up dgrad), then the SwiGLU backward and <G, a> as a row pass
    bf16_t* G = (bf16_t*)dXp;
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = (const bf16_t*)dout; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.B = (const bf16_t*)a.w_down; p.b_estride = d * I; p.ldb = I;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, TBN);
    p.row_major = rows_tile_order(a.T * d, a.E * d * I);
    p.C = G; p.ldc = I;
    err = launch_rows<EPI_STORE, B_KM, 1>(c, "gemm_down_dgrad", p, a.R, a.persistent);
    if (err != hipSuccess) return err;
    err = launch_swiglu_bwd(c, G, H, a.topk_w, a.src_of, a.R, a.I, a.swiglu_lim, dH, dwp);
    if (err != hipSuccess) return err;
  }
  {  // down wgrad: dW_d[e][c, i] = sum_r dout[t_r, c] Aw[r, i]
    WgradArgs p = {};
    p.A = (const bf16_t*)dout; p.lda = d; p.tok = a.tok_of;
    p.B = (const bf16_t*)Aw; p.ldb = I; p.E = a.E;
    p.M = a.d; p.N = a.I; p.m_tiles = (int)cdiv(a.d, TBM); p.n_tiles = (int)cdiv(a.I, TBN);
    p.offsets = a.offsets; p.xorder = a.xorder;
    p.C = (bf16_t*)dW_d; p.c_estride = d * I;
    err = launch_wgrad<0>(c, "gemm_down_wgrad", p, a.E, a.persistent);
    if (err != hipSuccess) return err;
  }
  {  // gate/up dgrad: dXp = dH W_gate_up[e]
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.tiles = a.tiles; p.E = a.E;
    p.A = (const bf16_t*)dH; p.lda = 2 * I; p.a_src = nullptr; p.a_div = 1;
    p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
    p.N = a.d; p.K = 2 * a.I; p.n_tiles = (int)cdiv(a.d, TBN);
    p.row_major = rows_tile_order(a.R * 2 * I, a.E * 2 * I * d);
    p.C = (bf16_t*)dXp; p.ldc = d;
    err = launch_rows<EPI_STORE, B_KM>(c, "gemm_gateup_dgrad", p, a.R, a.persistent);
    if (err != hipSuccess) return err;
  }
  {  // gate/up wgrad: dW_gu[e][j, c] = sum_r dH[r, j] x[t_r, c]
    WgradArgs p = {};
    p.A = (const bf16_t*)dH; p.lda = 2 * I; p.tok = a.tok_of;
    p.B = (const bf16_t*)a.x; p.ldb = d; p.E = a.E;
    p.M = 2 * a.I; p.N = a.d; p.m_tiles = (int)cdiv(2 * a.I, TBM); p.n_tiles = (int)cdiv(a.d, TBN);
    p.offsets = a.offsets; p.xorder = a.xorder;
    p.C = (bf16_t*)dW_gu; p.c_estride = 2 * I * d;
    err = launch_wgrad<1>(c, "gemm_gateup_wgrad", p, a.E, a.persistent);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
