// Row passes of the layer: dispatch gather, combine (weighted sum of each
// token's k expert rows, returned to the token's original position), the
// input-gradient reduction, and the top-k-weight / router-logit gradients.
//
// Dispatch and combine are the steps that move tokens to their experts and
// bring the results back to their original positions ("Prime Intellect's
// Prime Mega MoE Trains Giant AI Models 55% Faster", section "Where MoE
// training loses time"; "Prime Intellect Fused MoE Kernel: 3.11x MoE
// Training Speed", section "What a mixture-of-experts layer actually does").
// All are HBM-bound copies/reductions: 16-byte vector accesses, one wave per
// row, float32 accumulation in a fixed (slot) order, no atomics.
#include "common.h"

namespace moe {
namespace {

template <typename T> struct Vec;  // 16-byte vector of T
template <> struct Vec<float> {
  static constexpr int N = 4;
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
};

template <typename T>
__device__ __forceinline__ void unpack(const uint4& v, float* f) {
  if constexpr (sizeof(T) == 4) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float* f) {
  uint4 v;
  if constexpr (sizeof(T) == 4) {
    v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
    v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
  } else {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    v.x = u[0]; v.y = u[1]; v.z = u[2]; v.w = u[3];
  }
  return v;
}

// xp[r] = x[src_of[r] / k]; one wave per row, 4 rows per block.
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ src_of, int R,
                                                      int k, int row_vecs, uint4* __restrict__ xp) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = src_of[r] / k;
  const uint4* src = x + t * row_vecs;
  uint4* dst = xp + (int64_t)r * row_vecs;
  for (int c = lane; c < row_vecs; c += kWave) dst[c] = src[c];
}

// out[t] = sum_j w[t,j] * rows[row_of[t*k+j]] (w == null: weight 1), float32
// sum in slot order, one rounding at the end.  One wave per token.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ rows,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, int Tn, int k,
                                                      int row_vecs, uint4* __restrict__ out) {
  constexpr int N = Vec<T>::N;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int32_t* ro = row_of + (int64_t)t * k;
  for (int c = lane; c < row_vecs; c += kWave) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    int j = 0;
    for (; j + 4 <= k; j += 4) {  // four rows in flight, summed in slot order
      uint4 v[4];
      float s[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = rows[(int64_t)ro[j + q] * row_vecs + c];
        s[q] = w ? w[(int64_t)t * k + j + q] : 1.0f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[N];
        unpack<T>(v[q], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += s[q] * f[i];
      }
    }
    for (; j < k; ++j) {
      float f[N];
      unpack<T>(rows[(int64_t)ro[j] * row_vecs + c], f);
      const float s = w ? w[(int64_t)t * k + j] : 1.0f;
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += s * f[i];
    }
    out[(int64_t)t * row_vecs + c] = pack<T>(acc);
  }
}

// Dispatch as a scatter, for rows of 64 * CPL 16-byte chunks: one wave per
// token reads its row once and writes it to the token's k expert-sorted
// rows (row_of), so x is read once instead of k times.  Same result as
// permute_kernel; stores are non-temporal (the copies are read later, by
// another kernel).
template <int CPL>
__global__ __launch_bounds__(256) void permute_scatter_kernel(const uint4* __restrict__ x,
                                                              const int32_t* __restrict__ row_of, int Tn,
                                                              int k, uint4* __restrict__ xp) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  constexpr int RV = 64 * CPL;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  u32x4v v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = *(const u32x4v*)(x + (int64_t)t * RV + c * 64 + lane);
  const int32_t* ro = row_of + (int64_t)t * k;
  for (int j = 0; j < k; ++j) {
    u32x4v* dst = (u32x4v*)(xp + (int64_t)ro[j] * RV + lane);
#pragma unroll
    for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(v[c], dst + c * 64);
  }
}

// Same sum with CPL 16-byte chunks per lane known at compile time (row width
// 64 * CPL chunks): every lane issues the loads of RB rows x CPL chunks
// before accumulating, so more of each token's rows are in flight.  Each
// expert row is read exactly once, so the loads are non-temporal: they do
// not evict lines that other kernels' operands reuse.
template <typename T, int CPL, int RB>
__global__ __launch_bounds__(256) void combine_wide_kernel(const uint4* __restrict__ rows,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ w, int Tn, int k,
                                                           uint4* __restrict__ out) {
  constexpr int N = Vec<T>::N;
  constexpr int RV = 64 * CPL;  // 16-byte chunks per row
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int32_t* ro = row_of + (int64_t)t * k;
  float acc[CPL][N];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[c][i] = 0.0f;
  typedef unsigned int u32x4l __attribute__((ext_vector_type(4)));
  int j = 0;
  for (; j + RB <= k; j += RB) {
    uint4 v[RB][CPL];
    float s[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const uint4* src = rows + (int64_t)ro[j + q] * RV + lane;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const u32x4l x = __builtin_nontemporal_load((const u32x4l*)(src + c * 64));
        v[q][c] = uint4{x[0], x[1], x[2], x[3]};
      }
      s[q] = w ? w[(int64_t)t * k + j + q] : 1.0f;
    }
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float f[N];
        unpack<T>(v[q][c], f);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[c][i] += s[q] * f[i];
      }
  }
  for (; j < k; ++j) {
    const uint4* src = rows + (int64_t)ro[j] * RV + lane;
    const float sj = w ? w[(int64_t)t * k + j] : 1.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float f[N];
      unpack<T>(src[c * 64], f);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[c][i] += sj * f[i];
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {  // streamed out: no L2 line kept for the output
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const uint4 v = pack<T>(acc[c]);
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, (u32x4v*)(out + (int64_t)t * RV + c * 64 + lane));
  }
}

// d_topk_w[t,j] = sum over the partial dot products of row row_of[t*k+j]
// (fixed order); dlogits[t,e] = w_e (dw_e - sum_j w_j dw_j) on the selected
// experts, 0 elsewhere.  One wave per token; lane j holds slot j's gradient,
// which the expert lanes pick up through shuffles.
template <typename LT>
__global__ __launch_bounds__(256) void topk_grad_kernel(const float* __restrict__ dwp, int nblk,
                                                        const int32_t* __restrict__ row_of,
                                                        const int32_t* __restrict__ ids,
                                                        const float* __restrict__ w, int Tn, int k,
                                                        int E, float* __restrict__ d_topk_w,
                                                        LT* __restrict__ dlogits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  float inner = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kWave) {
    const int j = j0 + lane;
    float dw = 0.0f, wj = 0.0f;
    if (j < k) {
      const float* p = dwp + (int64_t)row_of[(int64_t)t * k + j] * nblk;
      for (int b = 0; b < nblk; ++b) dw += p[b];
      d_topk_w[(int64_t)t * k + j] = dw;
      wj = w[(int64_t)t * k + j];
    }
    const int lim = min(kWave, k - j0);
    for (int q = 0; q < lim; ++q) inner += __shfl(wj * dw, q, kWave);
  }
  if (!dlogits) return;
  if (k <= kWave) {
    // lane j < k: slot j's expert and gradient (dw of slot j recomputed in
    // the same order as above, so bit-equal)
    int idj = -1;
    float gj = 0.0f;
    if (lane < k) {
      const int64_t r = row_of[(int64_t)t * k + lane];
      float dw = 0.0f;
      for (int b = 0; b < nblk; ++b) dw += dwp[r * nblk + b];
      idj = ids[(int64_t)t * k + lane];
      gj = w[(int64_t)t * k + lane] * (dw - inner);
    }
    for (int e0 = 0; e0 < E; e0 += kWave) {  // every lane runs every pass: the shuffles read live lanes
      const int e = e0 + lane;
      float g = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int id = __shfl(idj, j, kWave);
        const float gv = __shfl(gj, j, kWave);
        if (id == e) g = gv;
      }
      if (e < E) dlogits[(int64_t)t * E + e] = from_f32<LT>(g);
    }
    return;
  }
  for (int e = lane; e < E; e += kWave) {
    float g = 0.0f;
    for (int j = 0; j < k; ++j) {
      if (ids[(int64_t)t * k + j] == e) {
        const float wj = w[(int64_t)t * k + j];
        const int64_t r = row_of[(int64_t)t * k + j];
        float dw = 0.0f;
        for (int b = 0; b < nblk; ++b) dw += dwp[r * nblk + b];
        g = wj * (dw - inner);
      }
    }
    dlogits[(int64_t)t * E + e] = from_f32<LT>(g);
  }
}

// SwiGLU backward of one row per wave, from G = dout_t W_down[e] (bf16):
// a = silu(g) u, dw_r = <G, a> (the row's top-k-weight gradient), dA = w_r G,
// dH = (dA u s (1 + g (1 - s)), dA silu(g)) with s = sigmoid(g); with a
// clamp lim, g and u as clamped and no gradient through an active clamp.  Lane l
// handles the 8-column chunks l, l + 64, ...; the float32 dot product is
// reduced across the wave in a fixed order.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ G,
                                                         const uint4* __restrict__ H,
                                                         const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ src_of, int R,
                                                         int chunks, float lim, uint4* __restrict__ dH,
                                                         float* __restrict__ dw) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int lane = threadIdx.x & 63;
  const float wr = topk_w[src_of[r]];
  const uint4* Gr = G + (int64_t)r * chunks;
  const uint4* Hg = H + (int64_t)r * 2 * chunks;
  const uint4* Hu = Hg + chunks;
  uint4* dg_out = dH + (int64_t)r * 2 * chunks;
  uint4* du_out = dg_out + chunks;
  float part = 0.0f;
  for (int c = lane; c < chunks; c += kWave) {
    float gv[8], g[8], u[8], dg[8], du[8];
    unpack<bf16_t>(Gr[c], gv);
    unpack<bf16_t>(Hg[c], g);
    unpack<bf16_t>(Hu[c], u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float gc = clamp_gate(g[i], lim), uc = clamp_up(u[i], lim);
      const float sg = sigmoidf_(gc);
      const float a = gc * sg * uc;
      part += gv[i] * a;
      const float dA = wr * gv[i];
      dg[i] = g[i] <= lim ? dA * uc * sg * (1.0f + gc * (1.0f - sg)) : 0.0f;
      du[i] = fabsf(u[i]) <= lim ? dA * gc * sg : 0.0f;
    }
    dg_out[c] = pack<bf16_t>(dg);
    du_out[c] = pack<bf16_t>(du);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
  if (lane == 0) dw[r] = part;
}

}  // namespace

hipError_t launch_swiglu_bwd(const LaunchCtx& c, const void* G, const void* H, const float* topk_w,
                             const int32_t* src_of, int R, int I, float lim, void* dH, float* dw) {
  MOE_LAUNCH(c, "swiglu_bwd", swiglu_bwd_kernel, dim3((R + 3) / 4), dim3(256), 0, (const uint4*)G,
             (const uint4*)H, topk_w, src_of, R, I / 8, lim, (uint4*)dH, dw);
  return hipSuccess;
}

hipError_t launch_permute(const LaunchCtx& c, const char* name, int dtype, const void* x,
                          const int32_t* src_of, const int32_t* row_of,
                          int R, int k, int d, void* xp) {
  const int row_vecs = d * (dtype == F32 ? 4 : 2) / 16;
  const int T = R / k;
  if (row_vecs == 256) {
    MOE_LAUNCH(c, name, permute_scatter_kernel<4>, dim3((T + 3) / 4), dim3(256), 0, (const uint4*)x,
               row_of, T, k, (uint4*)xp);
    return hipSuccess;
  }
  if (row_vecs == 512) {
    MOE_LAUNCH(c, name, permute_scatter_kernel<8>, dim3((T + 3) / 4), dim3(256), 0, (const uint4*)x,
               row_of, T, k, (uint4*)xp);
    return hipSuccess;
  }
  MOE_LAUNCH(c, name, permute_kernel, dim3((R + 3) / 4), dim3(256), 0, (const uint4*)x,
             src_of, R, k, row_vecs, (uint4*)xp);
  return hipSuccess;
}

hipError_t launch_combine(const LaunchCtx& c, const char* name, int dtype, const void* rows,
                          const int32_t* row_of, const float* w, int T, int k, int d, void* out) {
  const int row_vecs = d * (dtype == F32 ? 4 : 2) / 16;
  const dim3 grid((T + 3) / 4);
  // eight rows in flight per lane where a row takes four chunks a lane, four
  // at eight chunks (register budget)
  if (dtype == BF16 && row_vecs == 256) {
    MOE_LAUNCH(c, name, (combine_wide_kernel<bf16_t, 4, 8>), grid, dim3(256), 0, (const uint4*)rows,
               row_of, w, T, k, (uint4*)out);
    return hipSuccess;
  }
  if (dtype == BF16 && row_vecs == 512) {
    MOE_LAUNCH(c, name, (combine_wide_kernel<bf16_t, 8, 4>), grid, dim3(256), 0, (const uint4*)rows,
               row_of, w, T, k, (uint4*)out);
    return hipSuccess;
  }
  if (dtype == F32)
    MOE_LAUNCH(c, name, combine_kernel<float>, dim3((T + 3) / 4), dim3(256), 0,
               (const uint4*)rows, row_of, w, T, k, row_vecs, (uint4*)out);
  else
    MOE_LAUNCH(c, name, combine_kernel<bf16_t>, dim3((T + 3) / 4), dim3(256), 0,
               (const uint4*)rows, row_of, w, T, k, row_vecs, (uint4*)out);
  return hipSuccess;
}

hipError_t launch_topk_grad(const LaunchCtx& c, const float* dwp, int nblk, const int32_t* row_of,
                            const int32_t* ids, const float* w, int T, int k, int E,
                            float* d_topk_w, void* dlogits, int logits_dtype) {
  if (logits_dtype == F32)
    MOE_LAUNCH(c, "topk_grad", topk_grad_kernel<float>, dim3((T + 3) / 4), dim3(256), 0, dwp,
               nblk, row_of, ids, w, T, k, E, d_topk_w, (float*)dlogits);
  else
    MOE_LAUNCH(c, "topk_grad", topk_grad_kernel<bf16_t>, dim3((T + 3) / 4), dim3(256), 0, dwp,
               nblk, row_of, ids, w, T, k, E, d_topk_w, (bf16_t*)dlogits);
  return hipSuccess;
}

namespace {
__global__ __launch_bounds__(256) void tok_of_kernel(const int32_t* __restrict__ src_of, int R, int k,
                                                     int32_t* __restrict__ tok) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < R) tok[r] = src_of[r] / k;
}
}  // namespace

hipError_t launch_tok_of(const LaunchCtx& c, const int32_t* src_of, int R, int k, int32_t* tok) {
  if (R <= 0) return hipSuccess;
  MOE_LAUNCH(c, "route_tok", tok_of_kernel, dim3((unsigned)cdiv(R, 256)), dim3(256), 0, src_of, R, k, tok);
  return hipSuccess;
}

}  // namespace moe
