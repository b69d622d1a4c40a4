// Grouped GEMMs of the expert MLPs in bf16 on gfx950 MFMA (fp32 accumulate).
//
// Each expert is a SwiGLU MLP: both expert linear layers plus SwiGLU
// ("Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed", section
// "What a mixture-of-experts layer actually does"; "Mario/overlap moe kernel
// integration", overview: "SwiGLU expert GEMMs").  Fusion keeps
// intermediates out of separate passes ("Prime Intellect's Prime Mega MoE
// Trains Giant AI Models 55% Faster", section "One kernel overlaps the
// pipeline"): the token gather is the A-operand load of the gate/up GEMM,
// SwiGLU is its epilogue, and the SwiGLU backward plus the top-k-weight
// partial dot products are the epilogue of the down dgrad GEMM.
//
// One kernel shape serves all six GEMMs: C[m,n] = sum_k A(m,k) B(n,k) on a
// 128x128 output tile, K in steps of 64, four waves each owning 64x64 as 2x2
// MFMA 32x32x16 tiles.  Operands are staged through registers into a
// double-buffered LDS tile laid out [row][k] (16-byte chunks XOR-swizzled),
// so the global loads of step k+1 are in flight while the MFMAs of step k
// run: for the gate/up GEMM that is the gather of the next K slice of the
// tile's token rows.
//   * ragged M (forward, dgrad): rows are an expert's segment of the sorted
//     rows; blockIdx -> (row tile, N tile) through the tile table.
//   * ragged K (weight gradients): K runs over an expert's rows; experts are
//     visited largest first.
#include "common.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, NTHR = 256;
constexpr int TILE_BYTES = 128 * BK * 2;  // one operand tile in LDS
static_assert(BM == kRowTile, "tile table is built for BM-row tiles");

// physical 16-byte chunk of logical chunk kc in row `row`
__device__ __forceinline__ int swz(int row, int kc) { return kc ^ ((row ^ (row >> 3)) & 7); }
__device__ __forceinline__ int lds_off(int row, int kc) { return row * (BK * 2) + swz(row, kc) * 16; }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// ---------------------------------------------------------------------------
// Operand loaders.  Each stages a 128 x BK tile of (row, k) elements into LDS
// as [row][k].
// ---------------------------------------------------------------------------

// K-contiguous rows with arbitrary row pointers (gathered token rows, an
// expert's weight rows): element (row, k) = ptr[row][k].
struct RowKLoader {
  const bf16_t* ptr[4];
  int kc, K;
  uint4 v[4];
  __device__ void load(int kt) {
    const int k = kt * BK + kc * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (k < K) ? *(const uint4*)(ptr[i] + k) : zero4();
  }
  __device__ void store(char* s) const {
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(s + lds_off(r0 + 32 * i, kc)) = v[i];
  }
};

// Operand whose tile rows are contiguous in memory, one memory row per k
// (element (row, k) = memory_row(k)[row]).  Each thread loads 8 rows x 4 k as
// four 16-byte vectors and transposes them into the [row][k] LDS layout.
// Derived loaders supply load(kt), which fills v[q] with the 8 rows of k
// group kg*4+q.
struct ColKLoader {
  int rg, kg;  // row group (8 rows), k group (4 k)
  uint4 v[4];
  __device__ void init() {
    rg = threadIdx.x & 15;
    kg = threadIdx.x >> 4;
  }
  __device__ void store(char* s) const {
    const uint32_t* w0 = (const uint32_t*)&v[0];
    const uint32_t* w1 = (const uint32_t*)&v[1];
    const uint32_t* w2 = (const uint32_t*)&v[2];
    const uint32_t* w3 = (const uint32_t*)&v[3];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int q = m >> 1;
      uint2 p;
      if (m & 1) {
        p.x = (w0[q] >> 16) | (w1[q] & 0xffff0000u);
        p.y = (w2[q] >> 16) | (w3[q] & 0xffff0000u);
      } else {
        p.x = (w0[q] & 0xffffu) | (w1[q] << 16);
        p.y = (w2[q] & 0xffffu) | (w3[q] << 16);
      }
      const int row = rg * 8 + m;
      *(uint2*)(s + lds_off(row, kg >> 1) + (kg & 1) * 8) = p;
    }
  }
};

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
  uint32_t* w = (uint32_t*)&v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16) * s;
    const float hi = __uint_as_float(w[i] & 0xffff0000u) * s;
    w[i] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
  }
  return v;
}

// ---------------------------------------------------------------------------
// Main loop: double-buffered LDS, one barrier per K step.
// ---------------------------------------------------------------------------
template <class LA, class LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int nk, char* smem,
                                         f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  char* sa[2] = {smem, smem + 2 * TILE_BYTES};
  char* sb[2] = {smem + TILE_BYTES, smem + 3 * TILE_BYTES};
  la.load(0);
  lb.load(0);
  la.store(sa[0]);
  lb.store(sb[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    const char* A = sa[cur];
    const char* B = sb[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8_t*)(A + lds_off(wm * 64 + i * 32 + (lane & 31), kc));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const bf16x8_t*)(B + lds_off(wn * 64 + j * 32 + (lane & 31), kc));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(sa[cur ^ 1]);
      lb.store(sb[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Row (M index inside the tile) of accumulator register r of MFMA tile i for
// this lane; the column is (lane & 31) + 32 * j within the wave's 64 columns.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Finds the expert whose row tiles contain tile `mt`: largest e with
// tile_off[e] <= mt (empty experts share their successor's offset).
__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int mt) {
  int lo = 0, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

enum Epi { EPI_STORE = 0, EPI_GATEUP = 1, EPI_DGRAD_SWIGLU = 2 };
enum BLayout { B_ROWS = 0, B_ROWS_GATEUP = 1, B_COLS = 2 };

struct RowsArgs {
  // A(row, k) = A[arow(row) * lda + k], arow = a_src ? a_src[row] / a_div : row
  const bf16_t* A;
  int64_t lda;
  const int32_t* a_src;
  int a_div;
  // B_ROWS:        B(n, k) = Be[n * ldb + k]
  // B_ROWS_GATEUP: B(n, k) = Be[wrow(n) * ldb + k], gate/up rows interleaved
  //                in 32-row blocks (even block: gate, odd block: up)
  // B_COLS:        B(n, k) = Be[k * ldb + n]
  const bf16_t* B;
  int64_t b_estride, ldb;
  int N, K, n_tiles;  // N: output columns (gate/up: gate columns I)
  const int32_t* offsets;
  const int32_t* tile_off;
  int E;
  // EPI_STORE
  bf16_t* C;
  int64_t ldc;
  // EPI_GATEUP: H [R,2I] (optional), Aout [R,I]
  bf16_t* H;
  bf16_t* Aout;
  int I;
  // EPI_DGRAD_SWIGLU: Hin [R,2I], weight of row = topk_w[src_of[row]],
  // dwp [R, nblk] partial <G, a>, dH [R,2I]
  const bf16_t* Hin;
  const float* topk_w;
  const int32_t* src_of;
  float* dwp;
  int nblk;
  bf16_t* dH;
};

template <int EPI, int BL>
__global__ __launch_bounds__(NTHR, 2) void rows_gemm_kernel(RowsArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int L = blockIdx.x;
  const int nt = L % p.n_tiles;
  const int mt = L / p.n_tiles;
  if (mt >= p.tile_off[p.E]) return;
  const int e = find_expert(p.tile_off, p.E, mt);
  const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
  const int m0 = seg0 + (mt - p.tile_off[e]) * BM;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  RowKLoader la;
  la.kc = tid & 7;
  la.K = p.K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = m0 + (tid >> 3) + 32 * i;
    if (r >= seg1) r = seg0;  // rows past the segment are computed but never stored
    const int64_t ar = p.a_src ? (int64_t)(p.a_src[r] / p.a_div) : (int64_t)r;
    la.ptr[i] = p.A + ar * p.lda;
  }
  const bf16_t* Be = p.B + (int64_t)e * p.b_estride;

  f32x16_t acc[2][2];
  const int nk = (int)cdiv(p.K, BK);
  if constexpr (BL == B_COLS) {
    struct Loader : ColKLoader {
      const bf16_t* base;
      int64_t ld;
      int n0, N, K;
      __device__ void load(int kt) {
        const int n = n0 + rg * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = kt * BK + kg * 4 + q;
          v[q] = (n < N && k < K) ? *(const uint4*)(base + (int64_t)k * ld + n) : zero4();
        }
      }
    } lb;
    lb.init();
    lb.base = Be;
    lb.ld = p.ldb;
    lb.n0 = nt * BN;
    lb.N = p.N;
    lb.K = p.K;
    mainloop(la, lb, nk, smem, acc);
  } else {
    RowKLoader lb;
    lb.kc = tid & 7;
    lb.K = p.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = (tid >> 3) + 32 * i;  // tile column; 32-column block i
      int wrow;
      if constexpr (BL == B_ROWS_GATEUP) {
        int gc = nt * 64 + (i >> 1) * 32 + (n & 31);
        if (gc >= p.I) gc = 0;
        wrow = (i & 1) ? p.I + gc : gc;
      } else {
        wrow = nt * BN + n;
        if (wrow >= p.N) wrow = 0;
      }
      lb.ptr[i] = Be + (int64_t)wrow * p.ldb;
    }
    mainloop(la, lb, nk, smem, acc);
  }

  // ------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = nt * BN + wn * 64 + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, i, r, lane);
          if (row < seg1) p.C[(int64_t)row * p.ldc + col] = f2bf(acc[i][j][r]);
        }
    }
  } else if constexpr (EPI == EPI_GATEUP) {
    // acc[i][0]: gate, acc[i][1]: up, for gate column gc
    const int gc = nt * 64 + wn * 32 + (lane & 31);
    if (gc < p.I) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, i, r, lane);
          if (row >= seg1) continue;
          const float g = acc[i][0][r], u = acc[i][1][r];
          const float a = g * sigmoidf_(g) * u;
          p.Aout[(int64_t)row * p.I + gc] = f2bf(a);
          if (p.H) {
            p.H[(int64_t)row * 2 * p.I + gc] = f2bf(g);
            p.H[(int64_t)row * 2 * p.I + p.I + gc] = f2bf(u);
          }
        }
    }
  } else {  // EPI_DGRAD_SWIGLU: acc = G = dout_t W_down[e] for column i
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cb = nt * BN + wn * 64 + j * 32;  // 32-column block start
      const int col = cb + (lane & 31);
      const bool cok = col < p.N;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, i, r, lane);
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
          // sum over the 32 columns held by lanes of the same half-wave
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
          if ((lane & 31) == 0 && rok && cb < p.N)
            p.dwp[(int64_t)row * p.nblk + (cb >> 5)] = part;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight gradients: dW[e][m, n] = sum over the expert's rows r of
// A(m, r) B(n, r); both operands have m / n contiguous in memory.
// ---------------------------------------------------------------------------
struct WgradArgs {
  // A(m, r) = A[arow(r) * lda + m] * (a_scale ? a_scale[src_of[r]] : 1)
  const bf16_t* A;
  int64_t lda;
  int a_tok;  // arow(r) = a_tok ? src_of[r] / k : r
  const float* a_scale;
  // B(n, r) = B[brow(r) * ldb + n]
  const bf16_t* B;
  int64_t ldb;
  int b_tok;
  int M, N, m_tiles, n_tiles, k;
  const int32_t* offsets;
  const int32_t* order;
  const int32_t* src_of;
  bf16_t* C;  // dW[e] = C + e * c_estride, row-major [M, N]
  int64_t c_estride;
};

struct GatherColLoader : ColKLoader {
  const bf16_t* base;
  int64_t ld;
  int tok, kdiv;
  const float* scale;
  const int32_t* src_of;
  int m0, M, seg0, len;
  __device__ void load(int kt) {
    const int m = m0 + rg * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kr = kt * BK + kg * 4 + q;
      uint4 x = zero4();
      if (kr < len && m < M) {
        const int r = seg0 + kr;
        int64_t row = r;
        if (tok || scale) {
          const int f = src_of[r];
          if (tok) row = f / kdiv;
          x = *(const uint4*)(base + row * ld + m);
          if (scale) x = scale_bf16x8(x, scale[f]);
        } else {
          x = *(const uint4*)(base + row * ld + m);
        }
      }
      v[q] = x;
    }
  }
};

__global__ __launch_bounds__(NTHR, 2) void wgrad_kernel(WgradArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int per = p.m_tiles * p.n_tiles;
  const int oi = blockIdx.x / per;
  const int rem = blockIdx.x % per;
  const int mt = rem / p.n_tiles, nt = rem % p.n_tiles;
  const int e = p.order[oi];
  const int seg0 = p.offsets[e];
  const int len = p.offsets[e + 1] - seg0;
  GatherColLoader la, lb;
  la.init();
  lb.init();
  la.base = p.A; la.ld = p.lda; la.tok = p.a_tok; la.kdiv = p.k; la.scale = p.a_scale;
  la.src_of = p.src_of; la.m0 = mt * BM; la.M = p.M; la.seg0 = seg0; la.len = len;
  lb.base = p.B; lb.ld = p.ldb; lb.tok = p.b_tok; lb.kdiv = p.k; lb.scale = nullptr;
  lb.src_of = p.src_of; lb.m0 = nt * BN; lb.M = p.N; lb.seg0 = seg0; lb.len = len;
  f32x16_t acc[2][2];
  mainloop(la, lb, (int)cdiv(len, BK), smem, acc);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  bf16_t* C = p.C + (int64_t)e * p.c_estride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = nt * BN + wn * 64 + j * 32 + (lane & 31);
    if (col >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mt * BM + acc_row(wm, i, r, lane);
        if (row < p.M) C[(int64_t)row * p.N + col] = f2bf(acc[i][j][r]);
      }
  }
}

constexpr size_t kSmem = 4 * TILE_BYTES;  // 2 stages x (A + B)

int max_row_tiles(int R, int E) { return R / BM + E; }

template <int EPI, int BL>
hipError_t launch_rows(const LaunchCtx& c, const char* name, const RowsArgs& p, int R) {
  dim3 grid((unsigned)((int64_t)max_row_tiles(R, p.E) * p.n_tiles));
  MOE_LAUNCH(c, name, (rows_gemm_kernel<EPI, BL>), grid, dim3(NTHR), kSmem, p);
  return hipSuccess;
}

}  // namespace

hipError_t bf16_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aact, void* Y) {
  const int64_t I = a.I, d = a.d;
  RowsArgs p = {};
  p.offsets = a.offsets;
  p.tile_off = a.tile_off;
  p.E = a.E;
  // gate/up GEMM, token rows gathered from x, SwiGLU epilogue
  p.A = (const bf16_t*)a.x; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
  p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
  p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, 64);
  p.H = (bf16_t*)H; p.Aout = (bf16_t*)Aact; p.I = a.I;
  hipError_t err = launch_rows<EPI_GATEUP, B_ROWS_GATEUP>(c, "gemm_gateup_fwd", p, a.R);
  if (err != hipSuccess) return err;
  // down GEMM: Y = A W_down[e]^T
  RowsArgs q = {};
  q.offsets = a.offsets; q.tile_off = a.tile_off; q.E = a.E;
  q.A = (const bf16_t*)Aact; q.lda = I; q.a_src = nullptr; q.a_div = 1;
  q.B = (const bf16_t*)a.w_down; q.b_estride = d * I; q.ldb = I;
  q.N = a.d; q.K = a.I; q.n_tiles = (int)cdiv(a.d, BN);
  q.C = (bf16_t*)Y; q.ldc = d;
  return launch_rows<EPI_STORE, B_ROWS>(c, "gemm_down_fwd", q, a.R);
}

hipError_t bf16_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout,
                          const void* H, const void* Aact, void* dH, void* dXp, float* dwp,
                          void* dW_gu, void* dW_d) {
  const int64_t I = a.I, d = a.d;
  hipError_t err;
  {  // down dgrad: G = dout_t W_down[e]; epilogue: dw partials, SwiGLU backward -> dH
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.E = a.E;
    p.A = (const bf16_t*)dout; p.lda = d; p.a_src = a.src_of; p.a_div = a.k;
    p.B = (const bf16_t*)a.w_down; p.b_estride = d * I; p.ldb = I;
    p.N = a.I; p.K = a.d; p.n_tiles = (int)cdiv(a.I, BN);
    p.Hin = (const bf16_t*)H; p.topk_w = a.topk_w; p.src_of = a.src_of;
    p.dwp = dwp; p.nblk = (int)cdiv(a.I, 32); p.dH = (bf16_t*)dH; p.I = a.I;
    err = launch_rows<EPI_DGRAD_SWIGLU, B_COLS>(c, "gemm_down_dgrad", p, a.R);
    if (err != hipSuccess) return err;
  }
  {  // down wgrad: dW_d[e][c, i] = sum_r (w_r dout[t_r, c]) A[r, i]
    WgradArgs p = {};
    p.A = (const bf16_t*)dout; p.lda = d; p.a_tok = 1; p.a_scale = a.topk_w;
    p.B = (const bf16_t*)Aact; p.ldb = I; p.b_tok = 0;
    p.M = a.d; p.N = a.I; p.m_tiles = (int)cdiv(a.d, BM); p.n_tiles = (int)cdiv(a.I, BN);
    p.k = a.k; p.offsets = a.offsets; p.order = a.order; p.src_of = a.src_of;
    p.C = (bf16_t*)dW_d; p.c_estride = d * I;
    MOE_LAUNCH(c, "gemm_down_wgrad", wgrad_kernel, dim3(a.E * p.m_tiles * p.n_tiles), dim3(NTHR),
               kSmem, p);
  }
  {  // gate/up dgrad: dXp = dH W_gate_up[e]
    RowsArgs p = {};
    p.offsets = a.offsets; p.tile_off = a.tile_off; p.E = a.E;
    p.A = (const bf16_t*)dH; p.lda = 2 * I; p.a_src = nullptr; p.a_div = 1;
    p.B = (const bf16_t*)a.w_gate_up; p.b_estride = 2 * I * d; p.ldb = d;
    p.N = a.d; p.K = 2 * a.I; p.n_tiles = (int)cdiv(a.d, BN);
    p.C = (bf16_t*)dXp; p.ldc = d;
    err = launch_rows<EPI_STORE, B_COLS>(c, "gemm_gateup_dgrad", p, a.R);
    if (err != hipSuccess) return err;
  }
  {  // gate/up wgrad: dW_gu[e][j, c] = sum_r dH[r, j] x[t_r, c]
    WgradArgs p = {};
    p.A = (const bf16_t*)dH; p.lda = 2 * I; p.a_tok = 0; p.a_scale = nullptr;
    p.B = (const bf16_t*)a.x; p.ldb = d; p.b_tok = 1;
    p.M = 2 * a.I; p.N = a.d; p.m_tiles = (int)cdiv(2 * a.I, BM); p.n_tiles = (int)cdiv(a.d, BN);
    p.k = a.k; p.offsets = a.offsets; p.order = a.order; p.src_of = a.src_of;
    p.C = (bf16_t*)dW_gu; p.c_estride = 2 * I * d;
    MOE_LAUNCH(c, "gemm_gateup_wgrad", wgrad_kernel, dim3(a.E * p.m_tiles * p.n_tiles),
               dim3(NTHR), kSmem, p);
  }
  return hipSuccess;
}

}  // namespace moe
