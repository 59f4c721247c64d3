// Shared host and device pieces of the 256 x 256-tile GEMM kernels (NVFP4 /
// INT8 activations in qgemm.hip, MX activations in qgemm_mx.hip): launch
// parameters, the split of a partial last wave of tiles into K slices, the
// deterministic reduce pass of those slices, and the output stores.
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
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
  // quantizing epilogue (MX GEMM only): the next linear's MX activation
  uint8_t* q_out;          // [M][N / 2] E2M1 or [M][N] E4M3 codes
  uint8_t* s_out;          // [M][N / 32] E8M0 scales
  uint32_t qflags;         // 4: GELU before the transform
  const uint16_t* gtab;    // the device's GELU table (qflags 4)
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

// Two fp32 -> packed bf16 by the hardware conversion (v_cvt_pk_bf16_f32,
// round to nearest even): one instruction per pair in the epilogue.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
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
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + (int64_t)row * p.ldy + col) =
          make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
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
// row's token scale times the weight tensor scale, MX (2) none, bf16
// activations (3, the W4A16 fallback) the weight tensor scale.
template <int AFMT>
__device__ __forceinline__ float row_alpha(const GemmParams& p, int row) {
  if constexpr (AFMT == 0) return p.a_ts[1] * p.w_ts[1];
  else if constexpr (AFMT == 1) return static_cast<const float*>(p.a_s)[row] * p.w_ts[1];
  else if constexpr (AFMT == 3) return p.w_ts[1];
  else return 1.0f;
}

// Whether a tile's bf16 outputs can leave through LDS as whole 16-byte
// chunks (stage_store_tile).
__device__ __forceinline__ bool staged_store_ok(const GemmParams& p) {
  return !p.out_f32 && (p.N % 8) == 0 && (p.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15u) == 0 &&
         (!p.bias || (reinterpret_cast<uintptr_t>(p.bias) & 15u) == 0);
}

// bf16 epilogue of a 256 x 256 tile through LDS.  The accumulators hold Y^T
// blocks (lane = one token row, 4 consecutive features per register group),
// so direct stores would write 16 bytes into each of 32 rows per
// instruction.  Instead each wave writes its 128 x 128 sub-tile, scaled,
// biased and rounded to bf16, to LDS (rows of 256 bytes, 16-byte chunk c of
// row r at chunk position c ^ (r & 15): conflict-free writes), reads it back
// as 16-byte row chunks and stores 4 whole 256-byte row segments per
// instruction, marked non-temporal: the output is written once and is far
// larger than the L2, so it should not evict the operand stripes the other
// tiles of the XCD are still reading.  ROUNDS: the sub-tile goes through LDS in that many parts
// (32 KB / ROUNDS per wave); the caller has finished every LDS read of the
// ring, and smem holds at least 4 x 32 KB / ROUNDS bytes.
template <int AFMT, int ROUNDS>
__device__ __forceinline__ void stage_store_tile(const GemmParams& p, const float16v (&acc)[4][4], uint8_t* smem,
                                                 int m0, int n0) {
  constexpr int IPR = 4 / ROUNDS;                       // 32-row blocks per round
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1, r32 = lane & 31, h = lane >> 5;
  uint8_t* reg = smem + wv * (32768 / ROUNDS);
  // HB: add the bias (zeros where there is none).  The NVFP4 and MX
  // kernels take a second copy without it for calls with no bias (its 64
  // registers made the MX epilogue spill); in the INT8 kernel, whose rows
  // each load their own scale, a second copy made it spill instead, so it
  // always adds.
  auto body = [&](auto has_bias) {
    constexpr bool HB = decltype(has_bias)::value;
    // bias of this lane's 64 columns: 32 j + 8 g + 4 h .. +3 (of the wave's 128)
    float4 bias[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bias[j][g] = HB && p.bias
                         ? *reinterpret_cast<const float4*>(p.bias + min(n0 + wn * 128 + 32 * j + 8 * g + 4 * h, p.N - 4))
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();   // every wave is past its last read of the ring
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
#pragma unroll
      for (int ii = 0; ii < IPR; ++ii) {
        const int i = rd * IPR + ii;
        const int lrow = 32 * ii + r32;                   // row within this round's part
        const float alpha = row_alpha<AFMT>(p, min(m0 + wm * 128 + 32 * i + r32, p.M - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v0 = acc[i][j][4 * g] * alpha, v1 = acc[i][j][4 * g + 1] * alpha;
            float v2 = acc[i][j][4 * g + 2] * alpha, v3 = acc[i][j][4 * g + 3] * alpha;
            if constexpr (HB) {
              const float4 b = bias[j][g];
              v0 = v0 + b.x; v1 = v1 + b.y; v2 = v2 + b.z; v3 = v3 + b.w;
            }
            const int c = (4 * j + g) ^ (lrow & 15);
            *reinterpret_cast<uint2*>(reg + lrow * 256 + 16 * c + 8 * h) = make_uint2(bf16_pair(v0, v1), bf16_pair(v2, v3));
          }
      }
      // the same wave reads back what it wrote (LDS operations of a wave run
      // in order).  Eight reads go out before their eight stores: each store
      // sits behind its bounds branch, and a read issued after the previous
      // store would wait out the LDS latency once per 16-byte chunk
      const int c = lane & 15;
      const int col = n0 + wn * 128 + 8 * c;
      const int row0 = m0 + wm * 128 + 32 * rd * IPR + (lane >> 4);
      uint16_t* const y0 = static_cast<uint16_t*>(p.y) + (int64_t)row0 * p.ldy + col;
      const int64_t rstep = 4 * p.ldy;                   // 4 rows per read
#pragma unroll
      for (int b8 = 0; b8 < IPR; ++b8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int lrow = 4 * (8 * b8 + u) + (lane >> 4);
          v[u] = *reinterpret_cast<const uint4*>(reg + lrow * 256 + 16 * (c ^ (lrow & 15)));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int it = 8 * b8 + u;
          if (row0 + 4 * it < p.M && col < p.N)
            __builtin_nontemporal_store(uint4v{v[u].x, v[u].y, v[u].z, v[u].w},
                                        reinterpret_cast<uint4v*>(y0 + it * rstep));
        }
      }
    }
  };
  if constexpr (AFMT == 0 || AFMT == 2) {
    if (p.bias) body(std::true_type{});
    else body(std::false_type{});
  } else {
    body(std::true_type{});
  }
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

// Work split of a pipelined call on `cus` compute units, K in stages of
// `bk` (128 for the 4/8-bit activations, 64 for bf16).  Whole waves of
// tiles go to the data-parallel kernel.  The tiles of a last, partial wave
// (all tiles when there are fewer than CUs) are split into `slices` K slices,
// at most one workgroup per CU in all, when that is estimated to finish
// sooner than a partial wave of whole tiles: a slice's stages plus about
// kSplitOverhead stages of pipeline fill, partial-sum traffic and the reduce
// pass, against nk.
constexpr int kSplitOverhead = 3;

inline void plan_pipe(GemmParams& p, int cus, int& dp_grid, int& sk_grid, int bk = BK) {
  p.tiles_m = (p.M + 255) / 256;
  p.tiles_n = (p.N + 255) / 256;
  p.nk = p.K / bk;
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
inline int cu_count() { return device_cu_count(kGemmMaxGrid); }

}  // namespace vdtq
