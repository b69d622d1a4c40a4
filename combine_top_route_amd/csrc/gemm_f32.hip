// Float32 expert GEMMs (storage dtype float32): the same six GEMMs as the
// bf16 path, as plain FMA tiles with unfused SwiGLU passes.  This path keeps
// float32 precision end to end (the MFMA path rounds operands to bf16).
#include "common.h"

namespace moe {
namespace {

constexpr int FBM = 128, FBN = 64, FBK = 16;
static_assert(kRowTile % FBM == 0, "a row tile of the tile table is whole FBM-row blocks");

__device__ __forceinline__ int find_expert_f(const int32_t* tile_off, int E, int mt) {
  int lo = 0, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// C[row, n] = sum_k A[arow(row) * lda + k] * B[e * bes + n * bsn + k * bsk]
// for the rows of each expert's segment; arow = a_src ? a_src[row] / a_div : row.
__global__ __launch_bounds__(256) void f32_rows_gemm(const float* __restrict__ A, int64_t lda,
                                                     const int32_t* __restrict__ a_src, int a_div,
                                                     const float* __restrict__ B, int64_t bes,
                                                     int64_t bsn, int64_t bsk, float* __restrict__ C,
                                                     int64_t ldc, int N, int K,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_off, int E,
                                                     int n_tiles) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const int nt = blockIdx.x % n_tiles, mt = blockIdx.x / n_tiles;
  if (mt >= tile_off[E]) return;
  const int e = find_expert_f(tile_off, E, mt);
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  const int n0 = nt * FBN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* Be = B + (int64_t)e * bes;
  for (int m0 = seg0 + (mt - tile_off[e]) * kRowTile;
       m0 < seg1 && m0 < seg0 + (mt - tile_off[e] + 1) * kRowTile; m0 += FBM) {
  float acc[8][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, row = q >> 4, kk = q & 15;
      int r = m0 + row;
      if (r >= seg1) r = seg0;
      const int64_t ar = a_src ? (int64_t)(a_src[r] / a_div) : (int64_t)r;
      As[kk][row] = (k0 + kk < K) ? A[ar * lda + k0 + kk] : 0.0f;
    }
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, n = q >> 4, kk = q & 15;
      const int col = n0 + n;
      Bs[kk][n] = (col < N && k0 + kk < K) ? Be[(int64_t)col * bsn + (int64_t)(k0 + kk) * bsk] : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < FBK; ++kk) {
      float a[8], b[4];
      for (int i = 0; i < 8; ++i) a[i] = As[kk][ty * 8 + i];
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
      for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + ty * 8 + i;
    if (row >= seg1) continue;
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < N) C[(int64_t)row * ldc + col] = acc[i][j];
    }
  }
  }
}

// dW[e][m, n] = sum over rows r of expert e of A(m, r) B(n, r), with
// A(m, r) = A[arow(r) * lda + m] * (a_scale ? a_scale[src_of[r]] : 1),
// B(n, r) = B[brow(r) * ldb + n]; arow/brow = token of r (src_of[r] / k) or r.
__global__ __launch_bounds__(256) void f32_wgrad(const float* __restrict__ A, int64_t lda, int a_tok,
                                                 const float* __restrict__ a_scale,
                                                 const float* __restrict__ B, int64_t ldb, int b_tok,
                                                 int M, int N, int m_tiles, int n_tiles, int k,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ order,
                                                 const int32_t* __restrict__ src_of,
                                                 float* __restrict__ C, int64_t c_estride) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const int per = m_tiles * n_tiles;
  const int e = order[blockIdx.x / per];
  const int rem = blockIdx.x % per, mt = rem / n_tiles, nt = rem % n_tiles;
  const int seg0 = offsets[e], len = offsets[e + 1] - seg0;
  const int m0 = mt * FBM, n0 = nt * FBN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[8][4] = {};
  for (int k0 = 0; k0 < len; k0 += FBK) {
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, kk = q >> 7, ml = q & 127;
      float v = 0.0f;
      if (k0 + kk < len && m0 + ml < M) {
        const int r = seg0 + k0 + kk, f = src_of[r];
        const int64_t row = a_tok ? (int64_t)(f / k) : (int64_t)r;
        v = A[row * lda + m0 + ml] * (a_scale ? a_scale[f] : 1.0f);
      }
      As[kk][ml] = v;
    }
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, kk = q >> 6, nl = q & 63;
      float v = 0.0f;
      if (k0 + kk < len && n0 + nl < N) {
        const int r = seg0 + k0 + kk;
        const int64_t row = b_tok ? (int64_t)(src_of[r] / k) : (int64_t)r;
        v = B[row * ldb + n0 + nl];
      }
      Bs[kk][nl] = v;
    }
    __syncthreads();
    for (int kk = 0; kk < FBK; ++kk) {
      float a[8], b[4];
      for (int i = 0; i < 8; ++i) a[i] = As[kk][ty * 8 + i];
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
      for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Ce = C + (int64_t)e * c_estride;
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + ty * 8 + i;
    if (row >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < N) Ce[(int64_t)row * N + col] = acc[i][j];
    }
  }
}

// Aw[r, i] = w_r * silu(H[r, i]) * H[r, I + i], w_r = topk_w[src_of[r]]
// (gate and up clamped at lim; +inf: none)
__global__ __launch_bounds__(256) void f32_swiglu_fwd(const float* __restrict__ H,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ src_of, int64_t R,
                                                      int I, float lim, float* __restrict__ Aout) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= R * I) return;
  const int64_t r = q / I;
  const int i = (int)(q % I);
  const float g = clamp_gate(H[r * 2 * I + i], lim), u = clamp_up(H[r * 2 * I + I + i], lim);
  Aout[q] = topk_w[src_of[r]] * (g / (1.0f + expf(-g)) * u);
}

// From G = dout_t W_down[e] (per row): dwp[r, b] = sum over the 128 columns of
// block b of G * silu(g) * u; dA = w_r G; dH = (dA u s (1 + g (1 - s)), dA silu(g))
// (g, u clamped at lim, no gradient through an active clamp).
__global__ __launch_bounds__(256) void f32_swiglu_bwd(const float* __restrict__ G,
                                                      const float* __restrict__ H,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ src_of, int64_t R,
                                                      int I, int nblk, float lim, float* __restrict__ dH,
                                                      float* __restrict__ dwp) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= R * nblk) return;
  const int64_t r = q / nblk;
  const int b = (int)(q % nblk);
  const float w = topk_w[src_of[r]];
  float part = 0.0f;
  for (int i = b * 128; i < min(I, b * 128 + 128); ++i) {
    const float Gv = G[r * I + i];
    const float g0 = H[r * 2 * I + i], u0 = H[r * 2 * I + I + i];
    const float g = clamp_gate(g0, lim), u = clamp_up(u0, lim);
    const float s = 1.0f / (1.0f + expf(-g));
    part += Gv * (g * s * u);
    const float dA = w * Gv;
    dH[r * 2 * I + i] = g0 <= lim ? dA * u * s * (1.0f + g * (1.0f - s)) : 0.0f;
    dH[r * 2 * I + I + i] = fabsf(u0) <= lim ? dA * g * s : 0.0f;
  }
  dwp[q] = part;
}

hipError_t rows_gemm(const LaunchCtx& c, const char* name, const LayerArgs& a, const float* A,
                     int64_t lda, const int32_t* a_src, int a_div, const float* B, int64_t bes,
                     int64_t bsn, int64_t bsk, float* C, int64_t ldc, int N, int K) {
  const int n_tiles = (int)cdiv(N, FBN);
  const int64_t blocks = (int64_t)(a.R / kRowTile + a.E) * n_tiles;
  MOE_LAUNCH(c, name, f32_rows_gemm, dim3((unsigned)blocks), dim3(256), 0, A, lda, a_src, a_div,
             B, bes, bsn, bsk, C, ldc, N, K, a.offsets, a.tile_off, a.E, n_tiles);
  return hipSuccess;
}

hipError_t wgrad(const LaunchCtx& c, const char* name, const LayerArgs& a, const float* A,
                 int64_t lda, int a_tok, const float* a_scale, const float* B, int64_t ldb,
                 int b_tok, int M, int N, float* C) {
  const int mt = (int)cdiv(M, FBM), nt = (int)cdiv(N, FBN);
  MOE_LAUNCH(c, name, f32_wgrad, dim3((unsigned)(a.E * mt * nt)), dim3(256), 0, A, lda, a_tok,
             a_scale, B, ldb, b_tok, M, N, mt, nt, a.k, a.offsets, a.order, a.src_of, C,
             (int64_t)M * N);
  return hipSuccess;
}

}  // namespace

int f32_dw_blocks(int I) { return (int)cdiv(I, 128); }

hipError_t f32_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aact, void* Y) {
  const int64_t I = a.I, d = a.d, R = a.R;
  hipError_t err = rows_gemm(c, "gemm_gateup_fwd", a, (const float*)a.x, d, a.src_of, a.k,
                             (const float*)a.w_gate_up, 2 * I * d, d, 1, (float*)H, 2 * I,
                             (int)(2 * I), a.d);
  if (err != hipSuccess) return err;
  MOE_LAUNCH(c, "swiglu_fwd", f32_swiglu_fwd, dim3((unsigned)cdiv(R * I, 256)), dim3(256), 0,
             (const float*)H, a.topk_w, a.src_of, R, a.I, a.swiglu_lim, (float*)Aact);
  if (!Y) return hipSuccess;  // the gate/up half alone (recomputation)
  return rows_gemm(c, "gemm_down_fwd", a, (const float*)Aact, I, nullptr, 1,
                   (const float*)a.w_down, d * I, I, 1, (float*)Y, d, a.d, a.I);
}

hipError_t f32_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout, const void* H,
                         const void* Aact, void* dH, void* dXp, float* dwp, void* dW_gu,
                         void* dW_d, float* G) {
  const int64_t I = a.I, d = a.d, R = a.R;
  const int nblk = f32_dw_blocks(a.I);
  // down dgrad: G[r, i] = sum_c dout[t_r, c] W_down[e][c, i]
  hipError_t err = rows_gemm(c, "gemm_down_dgrad", a, (const float*)dout, d, a.src_of, a.k,
                             (const float*)a.w_down, d * I, 1, I, G, I, a.I, a.d);
  if (err != hipSuccess) return err;
  MOE_LAUNCH(c, "swiglu_bwd", f32_swiglu_bwd, dim3((unsigned)cdiv(R * nblk, 256)), dim3(256), 0,
             (const float*)G, (const float*)H, a.topk_w, a.src_of, R, a.I, nblk, a.swiglu_lim,
             (float*)dH, dwp);
  // down wgrad: dW_d[e][c, i] = sum_r dout[t_r, c] Aw[r, i]  (Aw carries w_r)
  err = wgrad(c, "gemm_down_wgrad", a, (const float*)dout, d, 1, nullptr, (const float*)Aact, I,
              0, a.d, a.I, (float*)dW_d);
  if (err != hipSuccess) return err;
  // gate/up dgrad: dXp[r, c] = sum_j dH[r, j] W_gate_up[e][j, c]
  err = rows_gemm(c, "gemm_gateup_dgrad", a, (const float*)dH, 2 * I, nullptr, 1,
                  (const float*)a.w_gate_up, 2 * I * d, 1, d, (float*)dXp, d, a.d, (int)(2 * I));
  if (err != hipSuccess) return err;
  return wgrad(c, "gemm_gateup_wgrad", a, (const float*)dH, 2 * I, 0, nullptr,
               (const float*)a.x, d, 1, (int)(2 * I), a.d, (float*)dW_gu);
}

}  // namespace moe
