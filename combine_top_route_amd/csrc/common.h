// Shared definitions of the HIP kernels (gfx950) and the host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum DType { F32 = 0, BF16 = 1 };

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t u) { return __uint_as_float((uint32_t)u << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two floats -> packed bfloat16 pair (lo in bits 0..15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// Logistic function with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ----------------------------------------------------------------------------
// Host side: every launcher reports its kernel through `launched` so the API
// layer can time it (profiling) and check the launch status.
// ----------------------------------------------------------------------------
struct LaunchCtx {
  hipStream_t stream;
  // called before and after each kernel enqueue with the kernel's name
  void (*before)(const char* name, hipStream_t s);
  void (*after)(const char* name, hipStream_t s);
};

#define MOE_LAUNCH(ctx, name, kernel, grid, block, shmem, ...)                     \
  do {                                                                             \
    if ((ctx).before) (ctx).before(name, (ctx).stream);                            \
    hipLaunchKernelGGL(kernel, grid, block, shmem, (ctx).stream, __VA_ARGS__);     \
    hipError_t _e = hipGetLastError();                                             \
    if ((ctx).after) (ctx).after(name, (ctx).stream);                              \
    if (_e != hipSuccess) return _e;                                               \
  } while (0)

#define HIP_RET(...)                        \
  do {                                      \
    hipError_t _r = (__VA_ARGS__);          \
    if (_r != hipSuccess) return _r;        \
  } while (0)

// ---------------------------------------------------------------- routing
// Tile table sizes: row tiles of the grouped GEMMs (expert-aligned).
constexpr int kRowTile = 256;
// Flat entries handled by one wave in the counting sort.
constexpr int kSortChunk = 1024;

hipError_t launch_topk(const LaunchCtx& c, const void* logits, int logits_dtype, int T, int E,
                       int k, int32_t* ids, float* w);
// counts / offsets / permutation from ids. hist: [ceil(R/kSortChunk), E] int32 scratch.
hipError_t launch_sort(const LaunchCtx& c, const int32_t* ids, int T, int E, int k,
                       int32_t* hist, int32_t* counts, int32_t* offsets, int32_t* row_of,
                       int32_t* src_of);
// GEMM schedule from offsets: tile_off [E+1] (row tiles of kRowTile per expert,
// prefix-summed), order [E] (experts by descending row count, ties by id) and,
// when blk_off is not null, blk_off [E+1] (runs of kTokBlock rows per expert,
// prefix-summed: the token blocks of the fp8 weight-gradient operands).
constexpr int kTokBlock = 128;
// tiles (optional) [tile_off[E]]: per row tile {expert, first row, end of the
// expert's segment, 0}.
hipError_t launch_schedule(const LaunchCtx& c, const int32_t* offsets, int E, int32_t* tile_off,
                           int32_t* order, int32_t* blk_off, int4* tiles);
// Upper bound of the row-tile count.
inline int64_t max_row_tiles(int64_t R, int64_t E) { return R / kRowTile + E; }

// ---------------------------------------------------------------- row passes
hipError_t launch_permute(const LaunchCtx& c, const char* name, int dtype, const void* x,
                          const int32_t* src_of,
                          int R, int k, int d, void* xp);
// out[t] = sum_j (w ? w[t*k+j] : 1) * rows[row_of[t*k+j]]
hipError_t launch_combine(const LaunchCtx& c, const char* name, int dtype, const void* rows,
                          const int32_t* row_of, const float* w, int T, int k, int d, void* out);
// bf16 SwiGLU backward per row from G [R,I] and H [R,2I]: dH [R,2I] and the
// row's top-k-weight gradient dw [R] = <G, silu(g) u>.
hipError_t launch_swiglu_bwd(const LaunchCtx& c, const void* G, const void* H, const float* topk_w,
                             const int32_t* src_of, int R, int I, void* dH, float* dw);
// d_topk_w[t,j] = sum_b dwp[row_of[t*k+j]*nblk + b]; dlogits (optional).
hipError_t launch_topk_grad(const LaunchCtx& c, const float* dwp, int nblk, const int32_t* row_of,
                            const int32_t* ids, const float* w, int T, int k, int E,
                            float* d_topk_w, void* dlogits, int logits_dtype);

// ---------------------------------------------------------------- GEMMs
struct LayerArgs {
  int T, d, E, k, I, R;
  int dtype;
  const void* x;
  const void* w_gate_up;
  const void* w_down;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* src_of;
  const int32_t* row_of;
  const int32_t* tile_off;  // [E+1], kRowTile tiles
  const int4* tiles;        // [tile_off[E]] row-tile descriptors
  const int32_t* order;     // [E]
};

// Forward GEMMs write H [R,2I] (gate|up, may be null), Aw [R,I] = w_row *
// silu(gate) * up (each row already carries its top-k weight) and Yw [R,d] =
// Aw W_down^T, so the combine is a plain sum of each token's k rows.
// bf16 MFMA path.
hipError_t bf16_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aw, void* Yw);
// backward outputs dH [R,2I], dXp [R,d], dwp [R, bf16_dw_blocks(I)] fp32, dW_gu, dW_d.
hipError_t bf16_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout,
                          const void* H, const void* Aw, void* dH, void* dXp, float* dwp,
                          void* dW_gu, void* dW_d);

// Number of per-row partials of <G, a> that the down dgrad writes (dwp [R, n]).
int bf16_dw_blocks(int I);
int f32_dw_blocks(int I);

// float32 path (plain FMA kernels, unfused epilogues).  forward needs H.
hipError_t f32_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, void* H, void* Aw, void* Yw);
// backward needs G [R,I] fp32 scratch.
hipError_t f32_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const void* dout,
                         const void* H, const void* Aw, void* dH, void* dXp, float* dwp,
                         void* dW_gu, void* dW_d, float* G);

// ---------------------------------------------------------------- fp8 path
// Block quantisation to e4m3 (quant_fp8.hip).  rows: 1 x 128 blocks along the
// rows of src [rows, C]; weight: 128 x 128 blocks of W [E, N, K], written as
// [E, N, K] or transposed [E, K, N] (scales [E, N/128, K/128] or transposed);
// tok: 128-row runs of each expert's segment x 1 column, written transposed
// q [C, 128 nblk_max], s [C, nblk_max].
hipError_t launch_quant_rows(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                             int64_t rows, int C, uint8_t* q, float* s);
hipError_t launch_quant_weight(const LaunchCtx& c, const char* name, const void* W, int E, int N,
                               int K, uint8_t* q, float* s, uint8_t* qt, float* st);
hipError_t launch_quant_tok(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                            const int32_t* src_of, int kdiv, int C, const int32_t* offsets,
                            const int32_t* blk_off, int E, int nblk_max, uint8_t* q, float* s);

// fp8 path's SwiGLU backward row pass: as launch_swiglu_bwd, plus dH's 1x128
// e4m3 codes dhq [R,2I] and scales dhs [R,2I/128] (I % 128 == 0).
hipError_t launch_swiglu_bwd_fp8(const LaunchCtx& c, const void* G, const void* H,
                                 const float* topk_w, const int32_t* src_of, int R, int I, void* dH,
                                 float* dw, uint8_t* dhq, float* dhs);

// Transposed weight codes the fp8 forward leaves in `saved` for the backward.
struct Fp8Saved {
  uint8_t* wdtq; float* wdts;    // [E,I,d], [E,I/128,d/128]
  uint8_t* wgutq; float* wguts;  // [E,d,2I], [E,d/128,2I/128]
};
// Workspace of the fp8 forward: quantised x, weights and Aw with their scales.
struct Fp8Fwd {
  uint8_t* xq; float* xs;      // [T,d], [T,d/128]
  uint8_t* wguq; float* wgus;  // [E,2I,d], [E,2I/128,d/128]
  uint8_t* wdq; float* wds;    // [E,d,I], [E,d/128,I/128]
  uint8_t* awq; float* aws;    // [R,I], [R,I/128]
  Fp8Saved sv;                 // written when saving for the backward (else null)
};
// Workspace of the fp8 backward.  tqa/tsa and tqb/tsb hold the two
// token-blocked operands of one weight gradient at a time
// ([max(d,2I)] and [max(I,d)] rows of 128 nblk_max bytes).
struct Fp8Bwd {
  uint8_t* doutq; float* douts;  // [T,d], [T,d/128]
  Fp8Saved sv;                   // from the forward's saved buffer
  uint8_t* dhq; float* dhs;      // [R,2I], [R,2I/128]
  uint8_t* tqa; float* tsa;
  uint8_t* tqb; float* tsb;
  const int32_t* blk_off;        // [E+1]
  int nblk_max;
};
int fp8_dw_blocks(int I);
// Same outputs as the bf16 path; H and Aw are stored in bf16.
hipError_t fp8_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Fwd& q, void* H, void* Aw,
                         void* Yw);
hipError_t fp8_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Bwd& q, const void* dout,
                         const void* H, const void* Aw, void* dH, void* dXp, float* dwp, void* dW_gu,
                         void* dW_d);

}  // namespace moe
