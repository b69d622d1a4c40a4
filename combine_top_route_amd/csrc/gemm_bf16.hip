// Grouped GEMMs of the expert MLPs in bf16 on gfx950 MFMA (fp32 accumulate).
//
// Each expert is a SwiGLU MLP: both expert linear layers plus SwiGLU
// ("Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed", section
// "What a mixture-of-experts layer actually does"; "Mario/overlap moe kernel
// integration", overview: "SwiGLU expert GEMMs").  Fusion keeps
// intermediates out of separate passes ("Prime Intellect's Prime Mega MoE
// Trains Giant AI Models 55% Faster", section "One kernel overlaps the
// pipeline"): the token gather is the A-operand load of the gate/up GEMM,
// SwiGLU and the top-k weighting are its epilogue, and the SwiGLU backward
// plus the top-k-weight partial dot products are the epilogue of the down
// dgrad GEMM.
//
// Tile engine (all six GEMMs): C[m,n] = sum_k A(m,k) B(n,k) on a 128x256 or
// 256x128 output tile, K in steps of 64, four waves of 64x128 / 128x64, each
// a grid of MFMA 32x32x16 bf16 tiles.  Operands move global -> LDS with
// direct loads (global_load_lds_dwordx4, no register staging) into a
// three-stage ring: while the MFMAs consume stage k, the loads of stage k+2
// are in flight - for the gate/up GEMM those are the gathered token rows of
// the next K slice, the one-GPU analogue of computing on one token group
// while the next one moves.  One barrier per K step.
//
// LDS layouts: an operand whose rows are K-contiguous in memory is stored
// [row][64 k] and read with ds_read_b128; an operand whose rows are contiguous
// along M/N (the weights in the dgrads, both operands of the weight
// gradients) is stored [k][cols] and read with ds_read_b64_tr_b16, whose
// 16-lane transpose hands each lane four consecutive k of one column.  Both
// layouts are XOR-swizzled so the reads of one instruction hit distinct
// banks.
#include "common.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int NSTAGE = 3;
constexpr int NTHR = 256;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Source of the direct loads that fall outside an operand (K tail, columns
// past N, rows past an expert's segment in the weight gradients).
__device__ __attribute__((aligned(64))) uint8_t g_zero_page[64] = {0};

__device__ __forceinline__ void dma16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that does not drain outstanding global loads (a
// __syncthreads fence would wait for the whole ring).  The empty asm keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// [row][k] layout: 64 bf16 = 128 bytes per row, 16-byte chunks XOR-swizzled.
__device__ __forceinline__ int mk_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int mk_off(int row, int kc) { return row * 128 + ((kc ^ mk_swz(row)) << 4); }

// [k][cols] layout: 32-byte chunks XOR-swizzled by k-row so that the four
// rows read together by a 16-lane group, and the two column halves of a
// 32-column fragment, land in distinct bank ranges.
__device__ __forceinline__ int km_swz(int krow) { return ((krow & 3) << 1) ^ ((krow >> 1) & 1); }

// ---------------------------------------------------------------------------
// Operand with K-contiguous rows (row r at rowp(r), element k at rowp(r)[k]).
// ROWS x 64 tile; instruction q covers rows 8q..8q+7 (1 KB of LDS); wave w
// issues q = w, w+4, ...
// ---------------------------------------------------------------------------
template <int ROWS>
struct OpMK {
  static constexpr int NI = ROWS / 32;
  static constexpr int BYTES = ROWS * BK * 2;
  const bf16_t* rowp[NI];
  int koff[NI];  // element offset of this lane's logical 16-byte chunk
  int K;

  template <class F>
  __device__ void init(F rowp_of, int K_) {
    K = K_;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = w + 4 * i;
      const int row = 8 * q + (lane >> 3);
      rowp[i] = rowp_of(row);
      koff[i] = (((lane & 7) ^ mk_swz(row)) << 3);
    }
  }
  __device__ void issue(int kt, char* s) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = kt * BK + koff[i];
      const void* g = (k < K) ? (const void*)(rowp[i] + k) : (const void*)g_zero_page;
      dma16(g, s + (w + 4 * i) * 1024);
    }
  }
  __device__ static bf16x8_t frag(const char* s, int rb, int kk) {
    const int lane = threadIdx.x & 63;
    const int row = rb + (lane & 31);
    return *(const bf16x8_t*)(s + mk_off(row, kk * 2 + (lane >> 5)));
  }
};

// ---------------------------------------------------------------------------
// Operand with column-contiguous k-rows: element (col, k) = krow_ptr(k)[col].
// COLS x 64 tile stored [k][COLS]; instruction q covers k-rows q*RPI..
// ---------------------------------------------------------------------------
template <int COLS>
struct OpKM {
  static constexpr int RB = COLS * 2;       // bytes per k-row
  static constexpr int UPR = RB / 16;       // 16-byte units per k-row
  static constexpr int RPI = 1024 / RB;     // k-rows per instruction
  static constexpr int NI = BK / RPI / 4;   // instructions per wave per stage
  static constexpr int BYTES = COLS * BK * 2;
  int krow[NI];   // k-row (0..63) of this lane in instruction i
  int coff[NI];   // column offset of this lane's logical 16-byte unit
  int c0, N;

  __device__ void init(int c0_, int N_) {
    c0 = c0_;
    N = N_;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = w + 4 * i;
      const int kr = q * RPI + lane / UPR;
      const int p = lane % UPR;
      const int u = (((p >> 1) ^ km_swz(kr)) << 1) | (p & 1);
      krow[i] = kr;
      coff[i] = u * 8;
    }
  }
  // kptr(k) returns the k-row's base pointer or nullptr (row outside the operand).
  template <class F>
  __device__ void issue(int kt, char* s, F kptr) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bf16_t* p = kptr(kt * BK + krow[i]);
      const int c = c0 + coff[i];
      const void* g = (p && c < N) ? (const void*)(p + c) : (const void*)g_zero_page;
      dma16(g, s + (w + 4 * i) * 1024);
    }
  }
  __device__ static bf16x8_t frag(const char* s, int cb, int kk) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, sl = lane & 15;
    const int col = cb + (g & 1) * 16 + 4 * (sl & 3);
    const int kr0 = kk * 16 + (g >> 1) * 8 + (sl >> 2);
    const int kr1 = kr0 + 4;
    const int ch = col >> 4;
    const char* p0 = s + kr0 * RB + ((ch ^ km_swz(kr0)) << 5) + ((col & 15) << 1);
    const char* p1 = s + kr1 * RB + ((ch ^ km_swz(kr1)) << 5) + ((col & 15) << 1);
    s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p0);
    s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p1);
    s16x8_t c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, c);
  }
};

// ---------------------------------------------------------------------------
// Main loop.  2 x 2 waves; wave tile (BM/2) x (BN/2) as TM x TN MFMA 32x32.
// ---------------------------------------------------------------------------
template <int BM, int BN, class OA, class OB, class IA, class IB>
__device__ __forceinline__ void mainloop(const OA& oa, const OB& ob, IA issue_a, IB issue_b, int nk,
                                         char* smem, f32x16_t (&acc)[BM / 64][BN / 64]) {
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int ST = OA::BYTES + OB::BYTES;
  constexpr int L = OA::NI + OB::NI;
  const int wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  issue_a(0, smem);
  issue_b(0, smem + OA::BYTES);
  if (nk > 1) {
    issue_a(1, smem + ST);
    issue_b(1, smem + ST + OA::BYTES);
  }
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmcnt<L>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (kt + 2 < nk) {
      const int s2 = slot == 0 ? 2 : slot - 1;  // (kt + 2) % 3
      issue_a(kt + 2, smem + s2 * ST);
      issue_b(kt + 2, smem + s2 * ST + OA::BYTES);
    }
    const char* As = smem + slot * ST;
    const char* Bs = As + OA::BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = OA::frag(As, wm * (BM / 2) + i * 32, kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = OB::frag(Bs, wn * (BN / 2) + j * 32, kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    slot = slot == 2 ? 0 : slot + 1;
  }
}

// Row inside the wave tile of accumulator register r of MFMA tile i; the
// column is (lane & 31) + 32 * j.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Largest e with tile_off[e] <= mt (empty experts share their successor's offset).
__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int mt) {
  int lo = 0, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Work-group id -> logical tile id.  Work-groups are dealt to the 8 XCDs
// round-robin; XCD x takes the x-th contiguous eighth of the `real` tiles, so
// each XCD walks consecutive tiles of the same expert (its row tiles share
// weight tiles, its N tiles share token rows, all through that XCD's L2) and
// the eight XCDs get equal tile counts whatever the routing.  Returns -1 for
// a work-group with nothing to do.
__device__ __forceinline__ int xcd_tile(int bid, int real) {
  const int per = (real + 7) >> 3;
  const int idx = bid >> 3;
  if (idx >= per) return -1;
  const int L = (bid & 7) * per + idx;
  return L < real ? L : -1;
}

// ===========================================================================
// Ragged-M GEMMs: rows are an expert's segment of the expert-sorted rows.
// Tile 128 rows x 256 columns.
// ===========================================================================
constexpr int RBM = 128, RBN = 256;
static_assert(RBM == kRowTile, "tile table is built for 128-row tiles");

enum Epi { EPI_STORE = 0, EPI_GATEUP = 1, EPI_DGRAD_SWIGLU = 2 };
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
  const int32_t* offsets;
  const int32_t* tile_off;
  int E;
  // EPI_STORE: C [R, ldc]
  bf16_t* C;
  int64_t ldc;
  // EPI_GATEUP: H [R,2I] (optional), Aw [R,I] = w_row * silu(g) * u
  bf16_t* H;
  bf16_t* Aout;
  int I;
  const float* topk_w;
  const int32_t* src_of;
  // EPI_DGRAD_SWIGLU: Hin [R,2I]; dwp [R, nblk] partial <G, silu(g) u>;
  // dH [R,2I]; weight of row = topk_w[src_of[row]]
  const bf16_t* Hin;
  float* dwp;
  int nblk;
  bf16_t* dH;
};

template <int EPI, int BL>
__global__ __launch_bounds__(NTHR, 1) void rows_gemm_kernel(RowsArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int L = xcd_tile(blockIdx.x, p.tile_off[p.E] * p.n_tiles);
  if (L < 0) return;
  const int nt = L % p.n_tiles;
  const int mt = L / p.n_tiles;
  const int e = find_expert(p.tile_off, p.E, mt);
  const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
  const int m0 = seg0 + (mt - p.tile_off[e]) * RBM;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  OpMK<RBM> oa;
  oa.init([&](int row) {
    int r = m0 + row;
    if (r >= seg1) r = seg0;  // rows past the segment: computed, never stored
    const int64_t ar = p.a_src ? (int64_t)(p.a_src[r] / p.a_div) : (int64_t)r;
    return p.A + ar * p.lda;
  }, p.K);
  const bf16_t* Be = p.B + (int64_t)e * p.b_estride;
  auto issue_a = [&](int kt, char* s) { oa.issue(kt, s); };

  f32x16_t acc[RBM / 64][RBN / 64];
  const int nk = (int)cdiv(p.K, BK);
  if constexpr (BL == B_KM) {
    OpKM<RBN> ob;
    ob.init(nt * RBN, p.N);
    const int K = p.K;
    const int64_t ldb = p.ldb;
    auto issue_b = [&](int kt, char* s) {
      ob.issue(kt, s, [&](int k) { return k < K ? Be + (int64_t)k * ldb : (const bf16_t*)nullptr; });
    };
    mainloop<RBM, RBN>(oa, ob, issue_a, issue_b, nk, smem, acc);
  } else {
    OpMK<RBN> ob;
    ob.init([&](int n) {
      int wrow;
      if constexpr (BL == B_MK_GATEUP) {
        const int blk = n >> 5;
        int gc = nt * (RBN / 2) + (blk >> 1) * 32 + (n & 31);
        if (gc >= p.I) gc = 0;
        wrow = (blk & 1) ? p.I + gc : gc;
      } else {
        wrow = nt * RBN + n;
        if (wrow >= p.N) wrow = 0;
      }
      return Be + (int64_t)wrow * p.ldb;
    }, p.K);
    auto issue_b = [&](int kt, char* s) { ob.issue(kt, s); };
    mainloop<RBM, RBN>(oa, ob, issue_a, issue_b, nk, smem, acc);
  }

  constexpr int TM = RBM / 64, TN = RBN / 64;
  const int rbase = m0 + wm * (RBM / 2);
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = nt * RBN + wn * (RBN / 2) + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + acc_row(i, r, lane);
          if (row < seg1) p.C[(int64_t)row * p.ldc + col] = f2bf(acc[i][j][r]);
        }
    }
  } else if constexpr (EPI == EPI_GATEUP) {
    // acc[i][2h] = gate, acc[i][2h+1] = up, gate column gc
#pragma unroll
    for (int h = 0; h < TN / 2; ++h) {
      const int gc = nt * (RBN / 2) + wn * (RBN / 4) + h * 32 + (lane & 31);
      if (gc >= p.I) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + acc_row(i, r, lane);
          if (row >= seg1) continue;
          const float g = acc[i][2 * h][r], u = acc[i][2 * h + 1][r];
          const float wr = p.topk_w[p.src_of[row]];
          p.Aout[(int64_t)row * p.I + gc] = f2bf(wr * (g * sigmoidf_(g) * u));
          if (p.H) {
            p.H[(int64_t)row * 2 * p.I + gc] = f2bf(g);
            p.H[(int64_t)row * 2 * p.I + p.I + gc] = f2bf(u);
          }
        }
    }
  } else {  // EPI_DGRAD_SWIGLU: acc = G = dout_t W_down[e] at column col
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cb = nt * RBN + wn * (RBN / 2) + j * 32;
      const int col = cb + (lane & 31);
      const bool cok = col < p.N;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + acc_row(i, r, lane);
          const bool rok = row < seg1;
          float part = 0.0f;
          if (rok && cok) {
            const float G = acc[i][j][r];
            const int64_t hb = (int64_t)row * 2 * p.I;
            const float g = bf2f(p.Hin[hb + col]);
            const float u = bf2f(p.Hin[hb + p.I + col]);
            const float wr = p.topk_w[p.src_of[row]];
            const float s = sigmoidf_(g);
            part = G * (g * s * u);
            const float dA = wr * G;
            p.dH[hb + col] = f2bf(dA * u * s * (1.0f + g * (1.0f - s)));
            p.dH[hb + p.I + col] = f2bf(dA * g * s);
          }
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
          if ((lane & 31) == 0 && rok && cb < p.N) p.dwp[(int64_t)row * p.nblk + (cb >> 5)] = part;
        }
    }
  }
}

// ===========================================================================
// Weight gradients: dW[e][m, n] = sum over the expert's rows r of
// A[seg0 + r][m] * B[seg0 + r][n]; both operands are row-major [R, *] with
// rows in expert order (contiguous per expert).  Tile 256 x 128.
// ===========================================================================
constexpr int WBM = 256, WBN = 128;

struct WgradArgs {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  int M, N, m_tiles, n_tiles;
  const int32_t* offsets;
  const int32_t* order;
  bf16_t* C;  // dW[e] = C + e * c_estride, row-major [M, N]
  int64_t c_estride;
};

__global__ __launch_bounds__(NTHR, 1) void wgrad_kernel(WgradArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int per = p.m_tiles * p.n_tiles;
  const int oi = blockIdx.x / per;
  const int rem = blockIdx.x % per;
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int e = p.order[oi];
  const int seg0 = p.offsets[e];
  const int len = p.offsets[e + 1] - seg0;
  OpKM<WBM> oa;
  OpKM<WBN> ob;
  oa.init(mt * WBM, p.M);
  ob.init(nt * WBN, p.N);
  const bf16_t* Ab = p.A + (int64_t)seg0 * p.lda;
  const bf16_t* Bb = p.B + (int64_t)seg0 * p.ldb;
  const int64_t lda = p.lda, ldb = p.ldb;
  auto issue_a = [&](int kt, char* s) {
    oa.issue(kt, s, [&](int k) { return k < len ? Ab + (int64_t)k * lda : (const bf16_t*)nullptr; });
  };
  auto issue_b = [&](int kt, char* s) {
    ob.issue(kt, s, [&](int k) { return k < len ? Bb + (int64_t)k * ldb : (const bf16_t*)nullptr; });
  };
  f32x16_t acc[WBM / 64][WBN / 64];
  mainloop<WBM, WBN>(oa, ob, issue_a, issue_b, (int)cdiv(len, BK), smem, acc);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  bf16_t* C = p.C + (int64_t)e * p.c_estride;
#pragma unroll
  for (int j = 0; j < WBN / 64; ++j) {
    const int col = nt * WBN + wn * (WBN / 2) + j * 32 + (lane & 31);
    if (col >= p.N) continue;
#pragma unroll
    for (int i = 0; i < WBM / 64; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mt * WBM + wm * (WBM / 2) + acc_row(i, r, lane);
        if (row < p.M) C[(int64_t)row * p.N + col] = f2bf(acc[i][j][r]);
      }
  }
}

constexpr size_t kRowsSmem = (size_t)NSTAGE * (RBM + RBN) * BK * 2;
constexpr size_t kWgradSmem = (size_t)NSTAGE * (WBM + WBN) * BK * 2;

template <class K>
hipError_t allow_smem(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int EPI, int BL>
hipError_t launch_rows(const LaunchCtx& c, const char* name, RowsArgs p, int R) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = allow_smem(rows_gemm_kernel<EPI, BL>, kRowsSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // upper bound of the tile count (the kernel reads the exact one)
  const int64_t tiles = (int64_t)(R / RBM + p.E) * p.n_tiles;
  const unsigned nblocks = (unsigned)((tiles + 7) / 8 * 8);
  MOE_LAUNCH(c, name, (rows_gemm_kernel<EPI, BL>), dim3(nblocks), dim3(NTHR), kRowsSmem, p);
  return hipSuccess;
}

hipError_t launch_wgrad(const LaunchCtx& c, const char* name, const WgradArgs& p, int E) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = allow_smem(wgrad_kernel, kWgradSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  MOE_LAUNCH(c, name, wgrad_kernel, dim3((unsigned)(E * p.m_tiles * p.n_tiles)), dim3(NTHR),
             kWgradSmem, p);
  return hipSuccess;
}

}  // namespace

hipError_t bf16_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aw, void* Yw) {
  const int64_t I = a.I, d = a.d;
  {  // gate/up GEMM: token rows gathered from x; SwiGLU and top-k weight in the epilogue
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.E = a.E;
    p.A = (const bf16_t*)a.x; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, RBN / 2);
    p.H = (bf16_t*)H; p.Aout = (bf16_t*)Aw; p.I = a.I;
    p.topk_w = a.topk_w; p.src_of = a.src_of;
    hipError_t err = launch_rows<EPI_GATEUP, B_MK_GATEUP>(c, "gemm_gateup_fwd", p, a.R);
    if (err != hipSuccess) return err;
  }
  // down GEMM: Yw = Aw W_down[e]^T (rows already carry their top-k weight)
  RowsArgs q = {};
  q.offsets = a.offsets; q.tile_off = a.tile_off; q.E = a.E;
  q.A = (const bf16_t*)Aw; q.lda = I; q.a_src = nullptr; q.a_div = 1;
  q.B = (const bf16_t*)a.w_down; q.b_estride = d * I; q.ldb = I;
  q.N = a.d; q.K = a.I; q.n_tiles = (int)cdiv(a.d, RBN);
  q.C = (bf16_t*)Yw; q.ldc = d;
  return launch_rows<EPI_STORE, B_MK>(c, "gemm_down_fwd", q, a.R);
}

hipError_t bf16_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout,
                          const void* H, const void* Aw, const void* Xp, const void* doutp,
                          void* dH, void* dXp, float* dwp, void* dW_gu, void* dW_d) {
  const int64_t I = a.I, d = a.d;
  hipError_t err;
  {  // down dgrad: G = dout_t W_down[e]; epilogue: dw partials, SwiGLU backward -> dH
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.E = a.E;
    p.A = (const bf16_t*)dout; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.B = (const bf16_t*)a.w_down; p.b_estride = d * I; p.ldb = I;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, RBN);
    p.Hin = (const bf16_t*)H; p.topk_w = a.topk_w; p.src_of = a.src_of;
    p.dwp = dwp; p.nblk = (int)cdiv(a.I, 32); p.dH = (bf16_t*)dH; p.I = a.I;
    err = launch_rows<EPI_DGRAD_SWIGLU, B_KM>(c, "gemm_down_dgrad", p, a.R);
    if (err != hipSuccess) return err;
  }
  {  // down wgrad: dW_d[e][c, i] = sum_r dout[t_r, c] Aw[r, i]
    WgradArgs p = {};
    p.A = (const bf16_t*)doutp; p.lda = d;
    p.B = (const bf16_t*)Aw; p.ldb = I;
    p.M = a.d; p.N = a.I; p.m_tiles = (int)cdiv(a.d, WBM); p.n_tiles = (int)cdiv(a.I, WBN);
    p.offsets = a.offsets; p.order = a.order;
    p.C = (bf16_t*)dW_d; p.c_estride = d * I;
    err = launch_wgrad(c, "gemm_down_wgrad", p, a.E);
    if (err != hipSuccess) return err;
  }
  {  // gate/up dgrad: dXp = dH W_gate_up[e]
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.E = a.E;
    p.A = (const bf16_t*)dH; p.lda = 2 * I; p.a_src = nullptr; p.a_div = 1;
    p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
    p.N = a.d; p.K = 2 * a.I; p.n_tiles = (int)cdiv(a.d, RBN);
    p.C = (bf16_t*)dXp; p.ldc = d;
    err = launch_rows<EPI_STORE, B_KM>(c, "gemm_gateup_dgrad", p, a.R);
    if (err != hipSuccess) return err;
  }
  {  // gate/up wgrad: dW_gu[e][j, c] = sum_r dH[r, j] x[t_r, c]
    WgradArgs p = {};
    p.A = (const bf16_t*)dH; p.lda = 2 * I;
    p.B = (const bf16_t*)Xp; p.ldb = d;
    p.M = 2 * a.I; p.N = a.d; p.m_tiles = (int)cdiv(2 * a.I, WBM); p.n_tiles = (int)cdiv(a.d, WBN);
    p.offsets = a.offsets; p.order = a.order;
    p.C = (bf16_t*)dW_gu; p.c_estride = 2 * I * d;
    err = launch_wgrad(c, "gemm_gateup_wgrad", p, a.E);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
