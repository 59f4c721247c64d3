// Shared device helpers of the GEMM kernels: direct-to-LDS loads with
// explicit waits, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdtq {

// Tile id -> coordinates: groups of 8 M-tiles, walked along N, so that tiles
// with neighbouring ids share A and W stripes.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int g = id / per_group;
  const int first_m = g * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in = id - g * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Workgroups are dealt round-robin to the 8 XCDs: give each XCD a
// contiguous range of ids, in dispatch order within the XCD.
__device__ __forceinline__ int xcd_range_id(int bid, int nblocks) {
  const int xcd = bid % 8, idx = bid / 8;
  const int base = nblocks / 8, rem = nblocks % 8;
  return xcd * base + min(xcd, rem) + idx;
}

typedef __attribute__((address_space(3))) void lds_void_t;

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The DMA is issued through inline asm so that the compiler's wait insertion,
// which cannot tell the ring slots apart, does not drain every in-flight load
// before each LDS read; the waits are explicit (wait_vm before the barrier).
// M0 holds the wave-uniform LDS destination (lane i writes M0 + i * size);
// the global address is a scalar base plus a 32-bit per-lane offset.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(m0), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               ::"s"(m0), "v"(voff), "s"(base) : "memory", "m0");
}

}  // namespace vdtq
