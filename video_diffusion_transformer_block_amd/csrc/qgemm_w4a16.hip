// W4A16: bf16 activations x NVFP4 weights, the full-precision fallback of a
// step whose input fails the outlier check (gist.science "6Bit-Diffusion:
// Inference-Time Mixed-Precision Quantization for Video Diffusion Models"
// §2.C: FP16/BF16 for that step; youleyou.com article §三).  The weights stay
// 4-bit ([gist] §4 memory figure); since they are stored rotated by the block
// Hadamard transform, the activations are the rotated ones (the BF16 output
// of hadamard_quantize).
//
// Arithmetic: every e2m1 * e4m3 weight value is exact in bf16 (at most 5
// significant bits, exponents 2^-10 .. 2^11), so W is decoded exactly and the
// product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; gs_w and
// the bias are applied in the epilogue.
//
// Data flow: one 256 x 256 output tile per 256-thread workgroup (4 waves,
// 2 x 2, each 128 x 128 = 4 x 4 MFMA tiles, accumulators holding Y^T tiles
// as in the NVFP4/INT8 kernels).  K in stages of 64 (a stage of A is 256 rows
// x 128 bytes of bf16), direct-to-LDS loads into a 3-deep ring issued two
// stages ahead, one barrier per stage.  Within a stage, lane half h and step
// s (0..3) cover k = 32 h + 8 s .. +8 for both operands: A is read as one
// 16-byte quad per row and step; W as one 16-byte quad (32 codes) per row and
// stage, decoded 8 codes per step: fp4 -> fp32 pairs (hardware conversion),
// times the group's E4M3 scale (exact), -> bf16 pairs.
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace vdtq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int A16_THREADS = 256;
constexpr int A16_BK = 64;
constexpr int A16_NS = 3;
constexpr int A16_A = 256 * 128;      // A bytes per stage
constexpr int A16_W = 256 * 32;       // W code bytes per stage
constexpr int A16_WS = 256 * 4;       // W scale bytes per stage
constexpr int A16_STAGE = A16_A + A16_W + A16_WS;
constexpr int A16_LPS = 8 + 2 + 1;    // loads per wave and stage

struct A16Params {
  const uint8_t* a;                   // bf16 [M][K]
  const uint8_t* w_q;
  const uint8_t* w_s;
  const float* w_ts;
  const float* bias;
  void* y;
  int64_t ldy;
  int32_t M, N, K;
  int32_t out_f32;
  int32_t tiles_m, tiles_n;
};

// LDS layout of a stage: A rows of 8 quads (16 B) stored at quad position
// q ^ (row & 7); W rows of 2 quads, unswizzled; W scales 4 bytes per row.
__device__ __forceinline__ int a16_quad_off(int row, int q) { return row * 128 + 16 * (q ^ (row & 7)); }

// 8 codes (one dword) times the group scale -> 8 exact bf16 values.
__device__ __forceinline__ bf16x8 dec_fp4x8_bf16(uint32_t w, float sc) {
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float2v f;
    switch (b) {
      case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    r[2 * b] = (__bf16)(f[0] * sc);
    r[2 * b + 1] = (__bf16)(f[1] * sc);
  }
  return r;
}

__global__ __launch_bounds__(A16_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm_a16_kernel(A16Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int r32 = lane & 31, h = lane >> 5;
  int tm, tn;
  tile_coords(xcd_range_id(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * 256, n0 = tn * 256;
  const int K = p.K;
  const int nk = K / A16_BK;

  // DMA sources at k0 = 0 (32-bit byte offsets, checked on the host)
  uint32_t offA[8], offW[2];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = (wv * 8 + u) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ (r & 7);
    offA[u] = (uint32_t)min(m0 + r, p.M - 1) * (uint32_t)(2 * K) + 16u * q;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = (wv * 2 + u) * 32 + (lane >> 1);
    offW[u] = (uint32_t)min(n0 + r, p.N - 1) * (uint32_t)(K / 2) + 16u * (lane & 1);
  }
  const uint32_t offWS = (uint32_t)min(n0 + wv * 64 + lane, p.N - 1) * (uint32_t)(K / 16);

  const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t*)smem;
  const uint32_t wvu = __builtin_amdgcn_readfirstlane(wv);
  auto issue_stage = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)(kt % A16_NS) * A16_STAGE;
    const int k0 = kt * A16_BK;
#pragma unroll
    for (int u = 0; u < 8; ++u) dma16(p.a + 2 * k0, offA[u], st + (wvu * 8 + u) * 1024);
#pragma unroll
    for (int u = 0; u < 2; ++u) dma16(p.w_q + k0 / 2, offW[u], st + A16_A + (wvu * 2 + u) * 1024);
    dma4(p.w_s + k0 / 16, offWS, st + A16_A + A16_W + wvu * 256);
  };

  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // this lane's W quads and group scales of a stage
  uint4 wq[4];
  float wsc[4][2];
  auto read_w = [&](int kt) {
    const uint8_t* st = smem + (kt % A16_NS) * A16_STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + 32 * j + r32;
      wq[j] = *reinterpret_cast<const uint4*>(st + A16_A + row * 32 + 16 * h);
      const uint32_t s4 = *reinterpret_cast<const uint32_t*>(st + A16_A + A16_W + row * 4);
      // steps 0-1 use group 2h, steps 2-3 group 2h + 1
      wsc[j][0] = e4m3_decode_pos((s4 >> (16 * h)) & 0xFFu);
      wsc[j][1] = e4m3_decode_pos((s4 >> (16 * h + 8)) & 0xFFu);
    }
  };
  // A fragments of step s read from LDS; W fragments decoded
  auto read_a = [&](int kt, int s, bf16x8 (&af)[4]) {
    const uint8_t* st = smem + (kt % A16_NS) * A16_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + r32;
      af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + a16_quad_off(row, 4 * h + s)));
    }
  };
  auto decode_w = [&](int s, bf16x8 (&bf)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = s == 0 ? wq[j].x : s == 1 ? wq[j].y : s == 2 ? wq[j].z : wq[j].w;
      bf[j] = dec_fp4x8_bf16(w, wsc[j][s >> 1]);
    }
  };
  auto mfma16 = [&](const bf16x8 (&af)[4], const bf16x8 (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
  };
  // each MFMA followed by a few VALU (decode) and, when present, one LDS read
  auto interleave = [&]() {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: stages 0..2 in flight, wait for stage 0
  issue_stage(0);
  if (nk > 1) issue_stage(1);
  if (nk > 2) issue_stage(2);
  if (nk > 2) wait_vm<2 * A16_LPS>();
  else if (nk > 1) wait_vm<A16_LPS>();
  else wait_vm<0>();
  wait_lgkm_barrier();

  bf16x8 fa[4], fb[4], ga[4], gb[4];
  read_w(0);
  read_a(0, 0, fa);
  decode_w(0, fb);

  // Every step has the same shape: the MFMAs of step s run beside the LDS
  // reads and W decode of step s+1.  The barrier sits before the last step:
  // by then every read of this stage's slot has been issued (lgkmcnt(0)), so
  // the slot takes the stage three ahead, and the next stage is complete, so
  // the last step can prepare its first.  Past the last stage those reads hit
  // a stale slot and are discarded.
  for (int kt = 0; kt < nk; ++kt) {
    // step 0 | step 1
    read_a(kt, 1, ga);
    decode_w(1, gb);
    mfma16(fa, fb);
    interleave();
    // step 1 | step 2
    read_a(kt, 2, fa);
    decode_w(2, fb);
    mfma16(ga, gb);
    interleave();
    // step 2 | step 3
    read_a(kt, 3, ga);
    decode_w(3, gb);
    mfma16(fa, fb);
    interleave();
    // stage kt+1 complete (only stage kt+2's loads may be in flight), every
    // wave done reading stage kt
    if (kt + 2 < nk) wait_vm<A16_LPS>();
    else wait_vm<0>();
    wait_lgkm_barrier();
    if (kt + 3 < nk) issue_stage(kt + 3);
    // step 3 | step 0 of stage kt+1
    read_w(kt + 1);
    read_a(kt + 1, 0, fa);
    decode_w(0, fb);
    mfma16(ga, gb);
    interleave();
  }

  // epilogue: tile (i, j), lane, register e -> token row m0 + wm*128 + 32 i
  // + lane%32, feature column n0 + wn*128 + 32 j + 8 (e/4) + 4 (lane/32) + e%4
  const float alpha = p.w_ts[1];
  const bool vec = (p.N % 4) == 0 && (p.ldy % 4) == 0 &&
                   ((reinterpret_cast<uintptr_t>(p.y) & (p.out_f32 ? 15u : 7u)) == 0) &&
                   (!p.bias || (reinterpret_cast<uintptr_t>(p.bias) & 15u) == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + 32 * i + r32;
    if (row >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * 128 + 32 * j + 8 * g + 4 * h;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q] * alpha;
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
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + (int64_t)row * p.ldy + col) =
                make_uint2(lo, hi);
          }
        } else {
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
      }
    }
  }
}

hipError_t launch_qgemm_w4a16(const void* a, const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M, int64_t N,
                              int64_t K, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  A16Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.w_q = w_q;
  p.w_s = w_s;
  p.w_ts = w_ts;
  p.bias = bias;
  p.y = y;
  p.ldy = ldy;
  p.M = (int32_t)M;
  p.N = (int32_t)N;
  p.K = (int32_t)K;
  p.out_f32 = out_dtype == 1;
  p.tiles_m = (int32_t)((M + 255) / 256);
  p.tiles_n = (int32_t)((N + 255) / 256);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemm_a16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, A16_NS * A16_STAGE);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(qgemm_a16_kernel, dim3(p.tiles_m * p.tiles_n), dim3(A16_THREADS),
                     (size_t)A16_NS * A16_STAGE, st, p);
  return hipGetLastError();
}

}  // namespace vdtq
