// Shared host and device pieces of the 256 x 256-tile GEMM kernels (NVFP4 /
// INT8 activations in qgemm.hip, MX activations in qgemm_mx.hip): launch
// parameters, the split of a partial last wave of tiles into K slices, the
// deterministic reduce pass of those slices, and the output stores.
#pragma once

#include <algorithm>

#include "device_common.h"
#include "lds_dma.h"

namespace vdtq {

constexpr int GT = 256;             // threads per workgroup
constexpr int kGemmMaxGrid = 256;   // pipelined path: at most one workgroup per CU
constexpr int BK = 128;             // K per stage

struct GemmParams {
  const void* a_q;
  const void* a_s;
  const float* a_ts;
  const uint8_t* w_q;
  const uint8_t* w_s;
  const float* w_ts;
  const float* bias;
  void* y;
  int64_t ldy;
  int32_t M, N, K;
  int32_t out_f32;
  int32_t tiles_m, tiles_n;
  // pipelined path: K stages per tile and the work split of the grid
  int32_t nk;
  int32_t sk_tiles;        // tiles 0 .. sk_tiles-1 are split along K
  int32_t slices;          // K slices per split tile (>= 2 when sk_tiles > 0)
  int32_t slice_nk;        // stages per slice (the last may be shorter)
  float* part;             // [slices][sk_tiles][256 * 256] partial tiles
};

// Partial tile of slice `sl` of split tile `tile`.  Layout inside a slot:
// [wave][64 float4][64 lanes], float4 q of a lane holding accumulator tile
// (q / 16, (q / 4) % 4), registers 4 (q % 4) .. 4 (q % 4) + 3.
__device__ __forceinline__ float4* part_slot(const GemmParams& p, int sl, int tile) {
  return reinterpret_cast<float4*>(p.part) + ((size_t)sl * p.sk_tiles + tile) * (256 * 256 / 4);
}

// LDS rows of packed codes, one stage (128 elements of K) per row.  4-bit
// rows: 64 bytes = 16-byte quads q = 0..3, stored at quad position
// q ^ ((row >> 1) & 3).  8-bit rows: 128 bytes = quads 0..7, stored at
// q ^ (row & 7).  The swizzle keeps the fragment reads (32 rows, one quad
// each) free of bank conflicts.
__device__ __forceinline__ int fp4_quad_off(int row, int q) { return row * 64 + 16 * (q ^ ((row >> 1) & 3)); }
__device__ __forceinline__ int i8_quad_off(int row, int q) { return row * 128 + 16 * (q ^ (row & 7)); }

// Whether four consecutive outputs of a row can go out as one vector store.
__device__ __forceinline__ bool out_vec_ok(const GemmParams& p) {
  return (p.N % 4) == 0 && (p.ldy % 4) == 0 &&
         ((reinterpret_cast<uintptr_t>(p.y) & (p.out_f32 ? 15u : 7u)) == 0) &&
         (!p.bias || (reinterpret_cast<uintptr_t>(p.bias) & 15u) == 0);
}

// Four consecutive outputs of one row: scale, bias, convert, store (columns
// past N are dropped).
__device__ __forceinline__ void emit4(const GemmParams& p, bool vec, int row, int col, float alpha, float x0,
                                      float x1, float x2, float x3) {
  float v[4] = {x0 * alpha, x1 * alpha, x2 * alpha, x3 * alpha};
  if (vec && col + 4 <= p.N) {
    if (p.bias) {
      const float4 b = *reinterpret_cast<const float4*>(p.bias + col);
      v[0] = v[0] + b.x; v[1] = v[1] + b.y; v[2] = v[2] + b.z; v[3] = v[3] + b.w;
    }
    if (p.out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.y) + (int64_t)row * p.ldy + col) =
          make_float4(v[0], v[1], v[2], v[3]);
    } else {
      const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + (int64_t)row * p.ldy + col) = make_uint2(lo, hi);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (col + q >= p.N) continue;
    float x = v[q];
    if (p.bias) x = x + p.bias[col + q];
    if (p.out_f32)
      static_cast<float*>(p.y)[(int64_t)row * p.ldy + col + q] = x;
    else
      static_cast<uint16_t*>(p.y)[(int64_t)row * p.ldy + col + q] = (uint16_t)f32_to_bf16_bits(x);
  }
}

// Output scale of a row: NVFP4 (AFMT 0) the two tensor scales, INT8 (1) the
// row's token scale times the weight tensor scale, MX (2) none.
template <int AFMT>
__device__ __forceinline__ float row_alpha(const GemmParams& p, int row) {
  if constexpr (AFMT == 0) return p.a_ts[1] * p.w_ts[1];
  else if constexpr (AFMT == 1) return static_cast<const float*>(p.a_s)[row] * p.w_ts[1];
  else return 1.0f;
}

// Split tiles: out = alpha * (sum of the slices in slice order) + bias.
// One thread per float4 of a partial slot; 64 workgroups per tile.
template <int AFMT>
__global__ __launch_bounds__(256) void qgemm_reduce_kernel(GemmParams p) {
  const int tile = (int)(blockIdx.x / 64);
  const int f = (int)(blockIdx.x % 64) * 256 + (int)threadIdx.x;   // float4 index in the slot
  const int wv = f >> 12, q = (f >> 6) & 63, lane = f & 63;
  const int i = q >> 4, j = (q >> 2) & 3, g = q & 3;
  int tm, tn;
  tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
  const int row = tm * 256 + (wv >> 1) * 128 + 32 * i + (lane & 31);
  const int col = tn * 256 + (wv & 1) * 128 + 32 * j + 8 * g + 4 * (lane >> 5);
  if (row >= p.M) return;
  float4 sum = part_slot(p, 0, tile)[f];
  for (int sl = 1; sl < p.slices; ++sl) {
    const float4 x = part_slot(p, sl, tile)[f];
    sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
  }
  emit4(p, out_vec_ok(p), row, col, row_alpha<AFMT>(p, row), sum.x, sum.y, sum.z, sum.w);
}

// Work split of a pipelined call on `cus` compute units.  Whole waves of
// tiles go to the data-parallel kernel.  The tiles of a last, partial wave
// (all tiles when there are fewer than CUs) are split into `slices` K slices,
// at most one workgroup per CU in all, when that is estimated to finish
// sooner than a partial wave of whole tiles: a slice's stages plus about
// kSplitOverhead stages of pipeline fill, partial-sum traffic and the reduce
// pass, against nk.
constexpr int kSplitOverhead = 3;

inline void plan_pipe(GemmParams& p, int cus, int& dp_grid, int& sk_grid) {
  p.tiles_m = (p.M + 255) / 256;
  p.tiles_n = (p.N + 255) / 256;
  p.nk = p.K / BK;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  const int G = std::max(1, std::min(cus, kGemmMaxGrid));
  const int64_t left = tiles % G;
  int slices = left > 0 ? (int)std::min<int64_t>(G / left, p.nk) : 0;
  int slice_nk = slices > 0 ? (p.nk + slices - 1) / slices : 0;
  if (slices > 0) slices = (p.nk + slice_nk - 1) / slice_nk;   // no empty slice
  const bool split = slices >= 2 && slice_nk + kSplitOverhead < p.nk;
  p.sk_tiles = split ? (int32_t)left : 0;
  p.slices = split ? slices : 0;
  p.slice_nk = split ? slice_nk : 0;
  dp_grid = (int)(tiles - p.sk_tiles);
  sk_grid = split ? (int)(left * slices) : 0;
}

// Compute units of the current device (cached per device).
inline int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kGemmMaxGrid;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kGemmMaxGrid;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace vdtq
