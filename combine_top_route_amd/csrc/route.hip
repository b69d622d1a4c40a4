// Routing kernels: top-k selection with renormalised softmax weights,
// per-expert counts and offsets, and the stable token sort into expert order.
//
// The router sends each token to a small subset of experts and the dispatch
// sorts tokens into expert order ("Prime Intellect's Prime Mega MoE Trains
// Giant AI Models 55% Faster", section "Where MoE training loses time"); the
// routing tensors are top scores, selected expert indices and per-expert
// token counts ("Mario/overlap moe kernel integration", commit on
// GroupedExperts.forward).
#include <climits>

#include "common.h"

namespace moe {
namespace {

// Monotone map float -> uint32 (larger float -> larger key). -0.0 is folded
// onto +0.0 first so that the two tie.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

constexpr int kMaxKeysPerLane = 1024 / kWave;  // E <= 1024

// One wavefront per token.  Key = ordered(logit) << 32 | ~expert, so the
// wave-wide maximum is the largest logit and, among equal logits, the lowest
// expert index.  k rounds of a wave arg-max; the winner's key is cleared.
template <typename LT>
__global__ __launch_bounds__(256) void topk_kernel(const LT* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const LT* row = logits + (int64_t)t * E;
  uint64_t key[kMaxKeysPerLane];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    int e = lane + kWave * i;
    key[i] = 0;
    if (e < E) {
      float v = to_f32<LT>(row[e]);
      key[i] = ((uint64_t)ordered_bits(v) << 32) | (uint32_t)(~(uint32_t)e);
    }
  }
  float my_logit = 0.0f;
  int my_id = 0;
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_u64(m);
    int e = (int)(~(uint32_t)(m & 0xffffffffu));
    float l = unordered_bits((uint32_t)(m >> 32));
    if (j == 0) top = l;
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kMaxKeysPerLane; ++i)
        if (i == (e >> 6)) key[i] = 0;
    }
    if (lane == j) {
      my_logit = l;
      my_id = e;
    }
  }
  // softmax over the k selected logits (float32), summed in slot order
  float ex = lane < k ? expf(my_logit - top) : 0.0f;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s += __shfl(ex, j, kWave);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = ex / s;
  }
}

// LPT lanes per token (adjacent lanes): lane p of a token walks the p-th
// contiguous E/LPT of its logits once and keeps the KMAX largest keys in a
// register list sorted descending (branch-free bubble insert); the LPT
// lists then merge pairwise through lane shuffles, each key of the partner's
// list inserted into one's own.  Keys are (ordered logit bits, ~expert), all
// distinct, so the merged list is the token's top KMAX whatever the split.
// Used for k <= KMAX; LPT > 1 needs E % (LPT * 16 bytes of logits) == 0.
template <typename LT, int KMAX, int LPT>
__global__ __launch_bounds__(256) void topk_lane_kernel(const LT* __restrict__ logits, int T, int E,
                                                        int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ w) {
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int t = gt / LPT, part = gt % LPT;
  // the token's LPT lanes exit together (t is shared), so the shuffles below
  // see only live partners
  if (t >= T) return;
  uint64_t top[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) top[j] = 0;
  auto insert = [&](uint64_t x) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const uint64_t hi = top[j] > x ? top[j] : x;
      x = top[j] > x ? x : top[j];
      top[j] = hi;
    }
  };
  auto push = [&](float v, int e) { insert(((uint64_t)ordered_bits(v) << 32) | (uint32_t)(~(uint32_t)e)); };
  const LT* row = logits + (int64_t)t * E;
  constexpr int VEC = 16 / sizeof(LT);
  if (LPT > 1 || (E % VEC == 0 && ((uintptr_t)logits & 15) == 0)) {
    const int span = E / LPT, e_lo = part * span;
    for (int e0 = e_lo; e0 < e_lo + span; e0 += VEC) {
      const uint4 v = *(const uint4*)(row + e0);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      if constexpr (sizeof(LT) == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) push(__uint_as_float(u[q]), e0 + q);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          push(__uint_as_float(u[q] << 16), e0 + 2 * q);
          push(__uint_as_float(u[q] & 0xffff0000u), e0 + 2 * q + 1);
        }
      }
    }
  } else {
    for (int e = 0; e < E; ++e) push(to_f32<LT>(row[e]), e);
  }
#pragma unroll
  for (int off = 1; off < LPT; off <<= 1) {
    uint64_t other[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const uint32_t lo = __shfl_xor((uint32_t)top[j], off, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(top[j] >> 32), off, 64);
      other[j] = ((uint64_t)hi << 32) | lo;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) insert(other[j]);
  }
  if (part != 0) return;
  // softmax over the k selected logits (float32), summed in slot order
  const float top0 = unordered_bits((uint32_t)(top[0] >> 32));
  float ex[KMAX];
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ex[j] = j < k ? expf(unordered_bits((uint32_t)(top[j] >> 32)) - top0) : 0.0f;
    s += ex[j];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      ids[(int64_t)t * k + j] = (int32_t)(~(uint32_t)(top[j] & 0xffffffffu));
      w[(int64_t)t * k + j] = ex[j] / s;
    }
  }
}

// Same selection for k > 64 (one lane per slot no longer fits a wave): the
// winners' logits and ids go through shared memory.
template <typename LT>
__global__ __launch_bounds__(64) void topk_kernel_bigk(const LT* __restrict__ logits, int T,
                                                       int E, int k, int32_t* __restrict__ ids,
                                                       float* __restrict__ w) {
  __shared__ float sl[1024];
  __shared__ int si[1024];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  if (t >= T) return;
  const LT* row = logits + (int64_t)t * E;
  uint64_t key[kMaxKeysPerLane];
#pragma unroll
  for (int i = 0; i < kMaxKeysPerLane; ++i) {
    int e = lane + kWave * i;
    key[i] = 0;
    if (e < E) key[i] = ((uint64_t)ordered_bits(to_f32<LT>(row[e])) << 32) | (uint32_t)(~(uint32_t)e);
  }
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_u64(m);
    int e = (int)(~(uint32_t)(m & 0xffffffffu));
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kMaxKeysPerLane; ++i)
        if (i == (e >> 6)) key[i] = 0;
      sl[j] = unordered_bits((uint32_t)(m >> 32));
      si[j] = e;
    }
  }
  __syncthreads();
  const float top = sl[0];
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s += expf(sl[j] - top);
  for (int j = lane; j < k; j += kWave) {
    ids[(int64_t)t * k + j] = si[j];
    w[(int64_t)t * k + j] = expf(sl[j] - top) / s;
  }
}

__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Histogram of one chunk of kSortChunk flat entries per block (one wave).
__global__ __launch_bounds__(64) void count_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                   int32_t* __restrict__ hist) {
  __shared__ int32_t h[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kSortChunk;
  for (int i = lane; i < kSortChunk; i += kWave) {
    int64_t f = base + i;
    if (f < R) atomicAdd(&h[clamp_id(ids[f], E)], 1);
  }
  __syncthreads();
  for (int e = lane; e < E; e += kWave) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// Block-wide exclusive scan of one value per thread (blockDim.x <= 1024).
__device__ int block_exclusive_scan(int v, int* sh_waves, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sh_waves[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    for (int i = 0; i < nw; ++i) {
      int tmp = sh_waves[i];
      sh_waves[i] = run;
      run += tmp;
    }
    *total = run;
  }
  __syncthreads();
  int r = sh_waves[wid] + incl - v;
  __syncthreads();
  return r;
}

// Per expert: prefix over chunks (hist becomes each chunk's start inside the
// expert's segment), counts, and offsets = exclusive scan of counts.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist, int nchunks, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int sh_waves[16];
  __shared__ int total;
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // loads of a batch are independent; only the running sum is serial
    for (int c0 = 0; c0 < nchunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (c0 + i < nchunks) ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < nchunks) hist[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
    counts[e] = run;
  }
  int off = block_exclusive_scan(e < E ? run : 0, sh_waves, &total);
  if (e < E) offsets[e] = off;
  if (e == 0) offsets[E] = total;
}

// Stable scatter: each wave walks its chunk in order, 64 entries at a time.
// Lanes routed to the same expert are found with one ballot per id bit; a
// lane's rank among them is the count of lower lanes in its match mask.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                     const int32_t* __restrict__ hist,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ row_of,
                                                     int32_t* __restrict__ src_of) {
  __shared__ int32_t base[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) base[e] = offsets[e] + hist[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t chunk0 = (int64_t)blockIdx.x * kSortChunk;
  for (int s = 0; s < kSortChunk; s += kWave) {
    const int64_t f = chunk0 + s + lane;
    const bool valid = f < R;
    const int e = valid ? clamp_id(ids[f], E) : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t mb = __ballot(bit);
      m &= bit ? mb : ~mb;
    }
    const int rank = __popcll(m & lt_mask);
    const int cnt = __popcll(m);
    int dest = 0;
    if (valid) dest = base[e] + rank;
    __syncthreads();
    if (valid) {
      row_of[f] = dest;
      src_of[dest] = (int32_t)f;
      if (rank == cnt - 1) base[e] = dest + 1;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int tiles_e(int rows) { return (rows + kRowTile - 1) / kRowTile; }

// Tile table of the grouped GEMMs and the expert order of the weight-gradient
// GEMMs (largest expert first, so the longest tiles start first).
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int E,
                                                        int32_t* __restrict__ tile_off,
                                                        int32_t* __restrict__ order,
                                                        int32_t* __restrict__ xorder,
                                                        int32_t* __restrict__ blk_off,
                                                        int4* __restrict__ tiles) {
  __shared__ int sh_waves[16];
  __shared__ int total;
  __shared__ int cnt[1024];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E) c = offsets[e + 1] - offsets[e];
  if (e < E) cnt[e] = c;
  int off = block_exclusive_scan(e < E ? tiles_e(c) : 0, sh_waves, &total);
  if (e < E) tile_off[e] = off;
  if (e == 0) tile_off[E] = total;
  if (tiles && e < E) {  // one descriptor per row tile: expert, first row, end of segment, expert's first tile
    const int seg0 = offsets[e], seg1 = offsets[e + 1];
    for (int t = 0; t < tiles_e(c); ++t) tiles[off + t] = make_int4(e, seg0 + t * kRowTile, seg1, off);
  }
  __syncthreads();
  if (blk_off) {
    const int blks = (c + kTokBlock - 1) / kTokBlock;
    const int boff = block_exclusive_scan(e < E ? blks : 0, sh_waves, &total);
    if (e < E) blk_off[e] = boff;
    if (e == 0) blk_off[E] = total;
    __syncthreads();
  }
  __shared__ int ord[1024];
  if (e < E) {
    int rank = 0;
    for (int o = 0; o < E; ++o) {
      int co = cnt[o];
      rank += (co > c) || (co == c && o < e);
    }
    order[rank] = e;
    ord[rank] = e;
  }
  __syncthreads();
  // Experts to XCDs for the weight gradients, where all tiles of an expert
  // run on one XCD: largest first, each to the least loaded XCD that has
  // fewer than ceil(E/8) experts (ties: lowest XCD).  An expert's cost is
  // its rows plus a fixed 192 for its tiles' prologue and epilogue.  Dealt
  // round-robin instead, a Zipf-skewed routing left the busiest XCD 26%
  // above the mean; this way it stays within about 2%.  Slot s of XCD x
  // lands at xorder[8 s + x] (-1: empty), as work-group 8 s + x runs on XCD
  // x.  Lane x of the first wave keeps XCD x's load and count in registers;
  // the experts go one at a time, to the lane that wins an argmin over the
  // eight lanes taken with DPP moves (the pass is serial, so each step
  // avoids the LDS round trip of a shuffle).
  if (xorder) {  // a kernel argument: uniform
    __shared__ int cost[1024];
    if (e < E) cost[e] = cnt[ord[e]] + 192;  // loads stay below R + 192 E < 2^28
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const int cap = (E + 7) / 8;
      int load = 0, n = 0;
      for (int c0 = 0; c0 < E; c0 += kWave) {
        // 64 experts' costs and ids in registers, taken lane by lane below
        const int cr = c0 + lane < E ? cost[c0 + lane] : 0;
        const int er = c0 + lane < E ? ord[c0 + lane] : 0;
        const int nn = E - c0 < kWave ? E - c0 : kWave;
        for (int j = 0; j < nn; ++j) {
          const int ci = __builtin_amdgcn_readlane(cr, j), ex = __builtin_amdgcn_readlane(er, j);
          // (load, lane) packed so that one integer min is the argmin
          // (loads stay below 2^28)
          int m = lane < 8 && n < cap ? load << 3 | lane : INT_MAX;
          m = min(m, __builtin_amdgcn_mov_dpp(m, 0xB1, 0xF, 0xF, false));   // lane ^ 1
          m = min(m, __builtin_amdgcn_mov_dpp(m, 0x4E, 0xF, 0xF, false));   // lane ^ 2
          m = min(m, __builtin_amdgcn_mov_dpp(m, 0x141, 0xF, 0xF, false));  // the other half of the eight
          if (lane < 8 && lane == (m & 7)) {
            xorder[n * 8 + lane] = ex;
            load += ci;
            ++n;
          }
        }
      }
      if (lane < 8)
        for (int slot = n; slot < cap; ++slot) xorder[slot * 8 + lane] = -1;
    }
  }
}

}  // namespace

hipError_t launch_topk(const LaunchCtx& c, const void* logits, int logits_dtype, int T, int E,
                       int k, int32_t* ids, float* w) {
  if (k <= 16) {
    // four lanes per token when each takes whole 16-byte runs of logits (and
    // the logits are 16-byte aligned), else one
    const int run = logits_dtype == F32 ? 4 : 8;
    const bool split = E % (4 * run) == 0 && ((uintptr_t)logits & 15) == 0;
    const dim3 grid((unsigned)cdiv((int64_t)T * (split ? 4 : 1), 256));
#define MOE_TOPK_LANE(LT, KM)                                                                     \
  do {                                                                                            \
    if (split)                                                                                    \
      MOE_LAUNCH(c, "route_topk", (topk_lane_kernel<LT, KM, 4>), grid, dim3(256), 0,              \
                 (const LT*)logits, T, E, k, ids, w);                                             \
    else                                                                                          \
      MOE_LAUNCH(c, "route_topk", (topk_lane_kernel<LT, KM, 1>), grid, dim3(256), 0,              \
                 (const LT*)logits, T, E, k, ids, w);                                             \
  } while (0)
    if (k <= 8) {
      if (logits_dtype == F32) MOE_TOPK_LANE(float, 8);
      else MOE_TOPK_LANE(bf16_t, 8);
    } else {
      if (logits_dtype == F32) MOE_TOPK_LANE(float, 16);
      else MOE_TOPK_LANE(bf16_t, 16);
    }
#undef MOE_TOPK_LANE
  } else if (k <= kWave) {
    dim3 grid((T + 3) / 4);
    if (logits_dtype == F32)
      MOE_LAUNCH(c, "route_topk", topk_kernel<float>, grid, dim3(256), 0, (const float*)logits, T,
                 E, k, ids, w);
    else
      MOE_LAUNCH(c, "route_topk", topk_kernel<bf16_t>, grid, dim3(256), 0, (const bf16_t*)logits,
                 T, E, k, ids, w);
  } else {
    if (logits_dtype == F32)
      MOE_LAUNCH(c, "route_topk", topk_kernel_bigk<float>, dim3(T), dim3(64), 0,
                 (const float*)logits, T, E, k, ids, w);
    else
      MOE_LAUNCH(c, "route_topk", topk_kernel_bigk<bf16_t>, dim3(T), dim3(64), 0,
                 (const bf16_t*)logits, T, E, k, ids, w);
  }
  return hipSuccess;
}

hipError_t launch_sort(const LaunchCtx& c, const int32_t* ids, int T, int E, int k, int32_t* hist,
                       int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of) {
  const int R = T * k;
  const int nchunks = (int)cdiv(R, kSortChunk);
  MOE_LAUNCH(c, "route_count", count_kernel, dim3(nchunks), dim3(64), 0, ids, R, E, hist);
  MOE_LAUNCH(c, "route_scan", scan_kernel, dim3(1), dim3(1024), 0, hist, nchunks, E, counts,
             offsets);
  MOE_LAUNCH(c, "route_scatter", scatter_kernel, dim3(nchunks), dim3(64), 0, ids, R, E, hist,
             offsets, row_of, src_of);
  return hipSuccess;
}

hipError_t launch_schedule(const LaunchCtx& c, const int32_t* offsets, int E, int32_t* tile_off,
                           int32_t* order, int32_t* xorder, int32_t* blk_off, int4* tiles) {
  MOE_LAUNCH(c, "route_schedule", schedule_kernel, dim3(1), dim3(1024), 0, offsets, E, tile_off,
             order, xorder, blk_off, tiles);
  return hipSuccess;
}

}  // namespace moe
