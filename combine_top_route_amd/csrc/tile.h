// Primitives shared by the MFMA tile engines (gfx950): LDS pointer types,
// direct global->LDS loads, wait/barrier helpers, the [row][128-byte] LDS
// swizzle and the mapping of work-groups to tiles.
#pragma once

#include <atomic>
#include <cstdint>

#include "common.h"

namespace moe {
namespace tile {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_t;  // byte pointer into LDS (32-bit)
typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16(const void* g, lds_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// Index of this thread's wave, as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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

// [row][k] layout: 128 bytes per row (64 bf16 or 128 fp8), 16-byte chunks
// XOR-swizzled so that 16 consecutive rows read at one chunk hit distinct banks.
__device__ __forceinline__ int mk_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int mk_off(int row, int kc) { return row * 128 + ((kc ^ mk_swz(row)) << 4); }

// 4-byte direct load (one float per lane).
__device__ __forceinline__ void dma4(const void* g, lds_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 4, 0, 0);
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

// Raises KERNEL's dynamic LDS limit to BYTES on the current device, once per
// device and kernel (attributes are per device; the bit set makes repeat
// launches free and is safe to race on: the call itself is idempotent).
template <auto KERNEL>
hipError_t allow_smem_once(size_t bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)KERNEL, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace tile
}  // namespace moe
