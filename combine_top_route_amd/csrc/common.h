// Shared definitions of the HIP kernels (gfx950) and the host launchers.
#pragma once

#include <hip/hip_ext.h>
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

// Clamped SwiGLU (DeepSeek V4's, as "Mario/overlap moe kernel integration"
// names it in its commit on activations.ClampedSilu): a = silu(min(g, lim))
// * clamp(u, -lim, lim).  lim = +inf gives the plain SwiGLU, bit for bit
// (min and max with +-inf leave finite values unchanged).  In the backward
// a gradient passes only where its clamp is inactive (at lim inclusive).
// One median-of-three each (v_med3_f32): fminf / fmaxf in IEEE mode cost a
// canonicalising max per operand on top of the min and max themselves.  The
// gate's lower bound -inf comes from an opaque move: with a literal -inf the
// compiler turns the median back into that min-with-canonicalise pair.
__device__ __forceinline__ float opaque_neg_inf() {
  float v;
  asm("s_mov_b32 %0, 0xff800000" : "=s"(v));
  return v;
}
__device__ __forceinline__ float clamp_gate(float g, float lim) {
  return __builtin_amdgcn_fmed3f(g, opaque_neg_inf(), lim);
}
__device__ __forceinline__ float clamp_up(float u, float lim) { return __builtin_amdgcn_fmed3f(u, -lim, lim); }

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Order of a row GEMM's tiles within an expert.  Either order re-reads one
// operand once per group of tiles that runs together: taken N-tile-major,
// the token rows (once per N tile); taken row-tile-major, the weight (once
// per group of row tiles).  The re-read operand should be the one that
// stays in the caches, the smaller: row-tile-major when the token operand's
// distinct bytes exceed the weight's (as for a GPU's expert-parallel share,
// few experts with many rows), else N-tile-major.
inline int rows_tile_order(int64_t token_bytes, int64_t weight_bytes) { return token_bytes > weight_bytes; }

// ----------------------------------------------------------------------------
// Host side: every launcher enqueues through MOE_LAUNCH, which checks the
// launch status and, while the API layer is timing kernels, hands the
// dispatch a start and a stop event: the runtime stamps them with the
// kernel's own start and end, with no extra packets on the stream.
// ----------------------------------------------------------------------------
struct LaunchCtx {
  hipStream_t stream;
  // while timing: the events to attach to the named kernel's dispatch (both
  // null when none are available)
  void (*events)(const char* name, hipEvent_t* start, hipEvent_t* stop);
};

#define MOE_LAUNCH(ctx, name, kernel, grid, block, shmem, ...)                               \
  do {                                                                                       \
    hipEvent_t _start = nullptr, _stop = nullptr;                                            \
    if ((ctx).events) (ctx).events(name, &_start, &_stop);                                   \
    if (_start)                                                                              \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, (ctx).stream, _start, _stop, 0,     \
                            __VA_ARGS__);                                                    \
    else                                                                                     \
      hipLaunchKernelGGL(kernel, grid, block, shmem, (ctx).stream, __VA_ARGS__);             \
    hipError_t _e = hipGetLastError();                                                       \
    if (_e != hipSuccess) return _e;                                                         \
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
constexpr int kMaxExperts = 1024;  // the C ABI rejects E outside [1, kMaxExperts]

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
// Per expert: row-tile offsets (tile_off, and tiles when non-null), order
// (experts by row count, largest first), xorder when non-null (the weight
// gradients' experts per XCD: slot s of XCD x at 8 s + x, -1 when empty; 8
// ceil(E/8) entries) and blk_off when non-null (128-row token blocks).
hipError_t launch_schedule(const LaunchCtx& c, const int32_t* offsets, int E, int32_t* tile_off,
                           int32_t* order, int32_t* xorder, int32_t* blk_off, int4* tiles);
// Upper bound of the row-tile count.
inline int64_t max_row_tiles(int64_t R, int64_t E) { return R / kRowTile + E; }

// ---------------------------------------------------------------- row passes
// xp[r] = x[src_of[r] / k]; rows of 4 or 8 KB are written as a scatter
// through row_of (x read once), others gathered through src_of.
hipError_t launch_permute(const LaunchCtx& c, const char* name, int dtype, const void* x,
                          const int32_t* src_of, const int32_t* row_of,
                          int R, int k, int d, void* xp);
// out[t] = sum_j (w ? w[t*k+j] : 1) * rows[row_of[t*k+j]]
hipError_t launch_combine(const LaunchCtx& c, const char* name, int dtype, const void* rows,
                          const int32_t* row_of, const float* w, int T, int k, int d, void* out);
// bf16 SwiGLU backward per row from G [R,I] and H [R,2I]: dH [R,2I] and the
// row's top-k-weight gradient dw [R] = <G, silu(g) u>.
// lim: the SwiGLU clamp (+inf: none).
hipError_t launch_swiglu_bwd(const LaunchCtx& c, const void* G, const void* H, const float* topk_w,
                             const int32_t* src_of, int R, int I, float lim, void* dH, float* dw);
// tok[r] = src_of[r] / k: the token of each expert-sorted row.
hipError_t launch_tok_of(const LaunchCtx& c, const int32_t* src_of, int R, int k, int32_t* tok);
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
  const int32_t* order;     // [E] experts by row count, largest first
  const int32_t* xorder;    // [8 ceil(E/8)] weight-gradient slot s of XCD x at 8 s + x (-1: empty)
  const int32_t* tok_of;    // [R] token of each sorted row (backward only)
  float swiglu_lim;         // SwiGLU clamp limit, +inf for the plain SwiGLU
  bool persistent;          // bf16 row GEMMs as persistent kernels
};

// Forward GEMMs write H [R,2I] (gate|up, may be null), Aw [R,I] = w_row *
// silu(gate) * up (each row already carries its top-k weight) and Yw [R,d] =
// Aw W_down^T, so the combine is a plain sum of each token's k rows.  Yw ==
// null: the gate/up GEMM alone (the recomputing backward).
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
// Block quantisation to e4m3 (quant_fp8.hip).  Two formats: blockwise (fp32
// scales; rows 1 x 128, weights 128 x 128, tokens 128-row runs) and MX
// (E8M0 scale bytes; rows 1 x 32, weights 1 x 32 along K and, transposed,
// along N, tokens 32-row blocks inside the 128-row runs).  Scale buffers are
// typed void*: fp32 values or E8M0 bytes.
//   rows:   src [rows, C] -> q [rows, C], s [rows, C/128] fp32 or [rows, C/32] bytes;
//           run_major: the 32-bit words [C/128, rows] instead; with row_of
//           (and k), the words [C/128, rows k] of the expert-sorted rows
//           row_of[r k + j] that gather token row r;
//   weight: W [E, N, K] -> q [E, N, K] and/or qt [E, K, N]; blockwise scales
//           s [E, N/128, K/128] / st [E, K/128, N/128]; MX s [E, N, K/32] /
//           st [E, K, N/32], or with run_major the words [E, K/128, N] /
//           [E, N/128, K];
//   tok:    128-row runs of each expert's segment, written transposed q [C,
//           128 nblk_max], one 32-bit scale word per run and column [C,
//           nblk_max] (an fp32 scale, or four E8M0 codes).
hipError_t launch_quant_rows(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                             int64_t rows, int C, uint8_t* q, void* s, bool mx, bool run_major,
                             const int32_t* row_of = nullptr, int k = 1);
hipError_t launch_quant_weight(const LaunchCtx& c, const char* name, const void* W, int E, int N,
                               int K, uint8_t* q, float* s, uint8_t* qt, float* st);
hipError_t launch_quant_weight_mx(const LaunchCtx& c, const char* name, const void* W, int E, int N,
                                  int K, uint8_t* q, uint8_t* s, uint8_t* qt, uint8_t* st, bool run_major);
// run_major: scale words [run][C] (as the weight-gradient GEMMs read them)
// instead of [C][nblk_max]
hipError_t launch_quant_tok(const LaunchCtx& c, const char* name, const void* src, int64_t ld,
                            const int32_t* src_of, int kdiv, int C, const int32_t* offsets,
                            const int32_t* blk_off, int E, int nblk_max, uint8_t* q, void* s,
                            bool mx, bool run_major);

// fp8 path's SwiGLU backward: from an fp32 G [R,I] and H, dH (bf16-rounded,
// never stored) in two e4m3 encodings: row codes dhq [R,2I] with scale words
// run-major dhs [2I/128, R], and the transposed token blocks of
// launch_quant_tok (run_major) in q / s; per-row partials of <G, a> into dw
// [R, I/128] (I % 128 == 0).
hipError_t launch_swiglu_bwd_tok(const LaunchCtx& c, const float* G, const void* H, const float* topk_w,
                                 const int32_t* src_of, int R, int I, float lim, const int32_t* offsets,
                                 const int32_t* blk_off, int E, int nblk_max, float* dw, uint8_t* dhq,
                                 void* dhs, uint8_t* q, void* s, bool mx);

// Weight codes the backward's data gradients read, left in `saved` by the
// fp8 forward: blockwise the forward encodings (one scale per 128 x 128
// block either way), MX the transposed encodings (blocks along the other
// axis).
struct Fp8Saved {
  uint8_t* wd_dgq; void* wd_dgs;    // codes and scales: blockwise [E,d,I], MX [E,I,d]
  uint8_t* wgu_dgq; void* wgu_dgs;  // blockwise [E,2I,d], MX [E,d,2I]
};
// Workspace of the fp8 forward: quantised x, weights and Aw with their scales.
struct Fp8Fwd {
  bool mx;                     // MXFP8 rather than blockwise
  uint8_t* xq; void* xs;       // codes [T,d]; scale words [d/128, R] per expert-sorted row
  uint8_t* wguq; void* wgus;   // [E,2I,d]
  uint8_t* wdq; void* wds;     // [E,d,I]
  uint8_t* awq; void* aws;     // codes [R,I]; scale words run-major [I/128, R]
  Fp8Saved sv;                 // written when saving for the backward (else null)
};
// Workspace of the fp8 backward.  tqa/tsa and tqb/tsb hold the two
// token-blocked operands of one weight gradient at a time
// ([max(d,2I)] and [max(I,d)] rows of 128 nblk_max bytes).
struct Fp8Bwd {
  bool mx;
  bool quant_weights;           // encode the weights into sv first
                                // (no fp8 forward ran)
  uint8_t* doutq; void* douts;  // codes [T,d]; scale words [d/128, R] per expert-sorted row
  Fp8Saved sv;                  // from the forward's saved buffer
  uint8_t* dhq; void* dhs;      // codes [R,2I]; scale words run-major [2I/128, R]
  uint8_t* tqa; void* tsa;
  uint8_t* tqb; void* tsb;
  float* G;                     // [R,I] the down dgrad's output
  const int32_t* blk_off;       // [E+1]
  int nblk_max;
};
int fp8_dw_blocks(int I);
// Same outputs as the bf16 path; H and Aw are stored in bf16.
hipError_t fp8_fwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Fwd& q, void* H, void* Aw,
                         void* Yw);
hipError_t fp8_bwd_gemms(const LaunchCtx& c, const LayerArgs& a, const Fp8Bwd& q, const void* dout,
                         const void* H, const void* Aw, void* dXp, float* dwp, void* dW_gu, void* dW_d);

}  // namespace moe
