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
// Data flow: the tile, work split, reduce pass and LDS-staged bf16 epilogue
// of the NVFP4/INT8 kernels (qgemm_common.h): one 256 x 256 output tile per
// 256-thread workgroup (4 waves, 2 x 2, each 128 x 128 = 4 x 4 MFMA tiles,
// accumulators holding Y^T tiles), whole waves of tiles data-parallel, the
// tiles of a partial last wave split into K slices.  K in stages of 64 (a
// stage of A is 256 rows x 128 bytes of bf16), direct-to-LDS loads into a
// 3-deep ring issued two stages ahead, one barrier per stage.  Within a
// stage, lane half h and step s (0..3) cover k = 32 h + 8 s .. +8 for both
// operands: A is read as one 16-byte quad per row and step; W as one 16-byte
// quad (32 codes) per row and stage, decoded 8 codes per step: fp4 -> fp32
// pairs (hardware conversion), times the group's E4M3 scale (exact), ->
// bf16 pairs (2 VALU per element: gfx950 has no packed bf16 multiply).
//
// W scales: with K % 256 == 0 (QUADS) a row's scale bytes of four
// consecutive stages are one 16-byte load per row, issued with every fourth
// stage into a double-buffered region past the ring (a scale load touches
// one row per lane: per-stage 4-byte loads cost as many memory requests as
// all the stage's A for an eighth of its bytes); otherwise 4 bytes per row
// with every stage.
//
// The main loop is scheduled by hand, as in qgemm.hip: each MFMA of a step
// is followed by one eighth of the next step's W decode (two elements) and
// at most one LDS read and one stage load, held together by sched_barrier.
// Reads: step 0 reads A of step 2, step 1 A of step 3; after the barrier,
// step 2 reads the next stage's W codes and scales and issues the loads of
// the stage three ahead, step 3 reads the next stage's A of steps 0 and 1.
#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "qgemm_common.h"

namespace vdtq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int A16_BK = 64;
constexpr int A16_NS = 3;
constexpr int A16_A = 256 * 128;      // A bytes per stage
constexpr int A16_W = 256 * 32;       // W code bytes per stage
constexpr int A16_WS = 256 * 4;       // W scale bytes per stage

template <bool QUADS>
struct A16Pipe {
  static constexpr int STAGE = A16_A + A16_W + (QUADS ? 0 : A16_WS);
  static constexpr int NLOAD = 8 + 2 + 1;           // load slots per wave and stage
  // loads per stage as the waits count them: with QUADS the scale slot
  // issues on every fourth stage only and is left out, so a wait for
  // "n stages in flight" is, if anything, stricter
  static constexpr int LPS = QUADS ? 8 + 2 : NLOAD;
  static constexpr int DUMMY = A16_NS * STAGE;      // landing area (1 KB per wave) of loads past the last stage
  static constexpr int SQ = DUMMY + 4096;           // scale quads: 2 buffers x 256 rows x 16 B
  static constexpr int END = SQ + (QUADS ? 2 * 4096 : 0);
  static constexpr int LDS = END > 4 * 32768 ? END : 4 * 32768;
};

// LDS layout of a stage: A rows of 8 quads (16 B) stored at quad position
// q ^ (row & 7); W rows of 2 quads, unswizzled; W scales 4 bytes per row.
__device__ __forceinline__ int a16_quad_off(int row, int q) { return row * 128 + 16 * (q ^ (row & 7)); }

template <bool SPLIT, bool QUADS>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm_a16_kernel(GemmParams p) {
  using P = A16Pipe<QUADS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int r32 = lane & 31, h = lane >> 5;
  const int K = p.K;
  const uint8_t* a_bf = static_cast<const uint8_t*>(p.a_q);

  int tile, kb, ke;
  if constexpr (SPLIT) {
    tile = (int)(blockIdx.x % p.sk_tiles);
    const int sl = (int)(blockIdx.x / p.sk_tiles);
    kb = sl * p.slice_nk;
    ke = min(p.nk, kb + p.slice_nk);
  } else {
    tile = p.sk_tiles + xcd_range_id(blockIdx.x, gridDim.x);
    kb = 0;
    ke = p.nk;
  }
  int tm, tn;
  tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * 256, n0 = tn * 256;

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
  auto ring = [&](int kt) { return (kt - kb) % A16_NS; };
  // Load u (0 .. NLOAD-1) of stage kt, branch-free: a stage past the last
  // reads the same 16 bytes (stage ke-1's base) in every lane into this
  // wave's landing area, one memory request instead of one per row.  The scale
  // slot with QUADS loads the 16 bytes of stages 4g .. 4g+3 per row into
  // buffer g % 2 on stage 4g (and on a slice's first stage), else nothing.
  const uint32_t dummy = lds0 + P::DUMMY + wvu * 1024;
  auto issue_one = [&](int kt, int u) {
    const uint32_t live = 0u - (uint32_t)(kt < ke);
    const int k0 = min(kt, ke - 1) * A16_BK;
    const uint32_t st = lds0 + (uint32_t)ring(kt) * P::STAGE;
    auto pick = [&](uint32_t target) { return dummy + ((target - dummy) & live); };
    if (u < 8) {
      dma16(a_bf + 2 * k0, offA[u] & live, pick(st + (wvu * 8 + u) * 1024));
    } else if (u < 10) {
      dma16(p.w_q + k0 / 2, offW[u - 8] & live, pick(st + A16_A + (wvu * 2 + (u - 8)) * 1024));
    } else if constexpr (QUADS) {
      if (kt < ke && ((kt & 3) == 0 || kt == kb))
        dma16(p.w_s + (kt >> 2) * 16, offWS, lds0 + P::SQ + (uint32_t)((kt >> 2) & 1) * 4096u + wvu * 1024u);
    } else {
      dma4(p.w_s + k0 / 16, offWS & live, pick(st + A16_A + A16_W + wvu * 256));
    }
  };
  auto issue_stage = [&](int kt) {
#pragma unroll
    for (int u = 0; u < P::NLOAD; ++u) issue_one(kt, u);
  };

  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // LDS reads of one fragment: A of step s, W codes, W scale dword (a lane's
  // two groups: steps 0-1 use group 2h, steps 2-3 group 2h + 1)
  auto read_a = [&](int kt, int s, int i, bf16x8& af) {
    const uint8_t* st = smem + ring(kt) * P::STAGE;
    af = __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const uint4*>(st + a16_quad_off(wm * 128 + 32 * i + r32, 4 * h + s)));
  };
  auto read_wq = [&](int kt, int j, uint4& q) {
    const uint8_t* st = smem + ring(kt) * P::STAGE;
    q = *reinterpret_cast<const uint4*>(st + A16_A + (wn * 128 + 32 * j + r32) * 32 + 16 * h);
  };
  auto read_ws = [&](int kt, int j, uint32_t& s4) {
    if constexpr (QUADS) {
      s4 = *reinterpret_cast<const uint32_t*>(smem + P::SQ + ((kt >> 2) & 1) * 4096 + (wn * 128 + 32 * j + r32) * 16 +
                                              4 * (kt & 3));
    } else {
      const uint8_t* st = smem + ring(kt) * P::STAGE;
      s4 = *reinterpret_cast<const uint32_t*>(st + A16_A + A16_W + (wn * 128 + 32 * j + r32) * 4);
    }
  };
  // group g's E4M3 scale as fp32: the hardware fp8 conversion (exact for
  // every E4M3 byte; no branch, which would split the step's schedule)
  auto scale_of = [&](uint32_t s4, int g) {
    const int v = (int)(s4 >> (16 * h));
    return g ? __builtin_amdgcn_cvt_f32_fp8(v, 1) : __builtin_amdgcn_cvt_f32_fp8(v, 0);
  };
  // elements 2b, 2b + 1 of W fragment j at step s (codes q, group scale sc)
  auto piece = [&](const uint4& q, float sc, int s, int b, bf16x8& out) {
    const uint32_t w = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
    float2v f;
    switch (b) {
      case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    out[2 * b] = (__bf16)(f[0] * sc);
    out[2 * b + 1] = (__bf16)(f[1] * sc);
  };
  auto step = [&](const bf16x8 (&CA)[4], const bf16x8 (&CB)[4], auto&& work) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CB[x & 3], CA[x >> 2], acc[x >> 2][x & 3], 0, 0, 0);
      work(x);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: stages kb..kb+2 in flight, wait for stage kb
  issue_stage(kb);
  issue_stage(kb + 1);
  issue_stage(kb + 2);
  wait_vm<2 * P::LPS>();
  wait_lgkm_barrier();

  bf16x8 A0[4], A1[4], A2[4], A3[4], B0[4], B1[4];
  uint4 wq[4], wqn[4];
  uint32_t ws4[4], ws4n[4];
  float sc0[4], sc1[4], sn0[4], sn1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    read_wq(kb, j, wq[j]);
    read_ws(kb, j, ws4[j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    read_a(kb, 0, i, A0[i]);
    read_a(kb, 1, i, A1[i]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc0[j] = scale_of(ws4[j], 0);
    sc1[j] = scale_of(ws4[j], 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) piece(wq[j], sc0[j], 0, b, B0[j]);
  }

  // Every stage has the same shape; past the last stage the reads of the
  // "next" stage hit a stale slot (or the loads' landing area) and the
  // extra decode is discarded.
  for (int kt = kb; kt < ke; ++kt) {
    // step 0 | W step 1; read A of step 2
    step(A0, B0, [&](int x) {
      piece(wq[x >> 2], sc0[x >> 2], 1, x & 3, B1[x >> 2]);
      if (x < 4) read_a(kt, 2, x, A2[x]);
    });
    // step 1 | W step 2; read A of step 3
    step(A1, B1, [&](int x) {
      piece(wq[x >> 2], sc1[x >> 2], 2, x & 3, B0[x >> 2]);
      if (x < 4) read_a(kt, 3, x, A3[x]);
    });
    // every read of stage kt is done and stage kt+1 has landed (only stage
    // kt+2's loads may be in flight): the slot takes stage kt+3
    wait_vm<P::LPS>();
    wait_lgkm_barrier();
    // step 2 | W step 3; stage kt+1's W scales and codes; loads of stage kt+3
    step(A2, B0, [&](int x) {
      piece(wq[x >> 2], sc1[x >> 2], 3, x & 3, B1[x >> 2]);
      if (x < 4) read_ws(kt + 1, x, ws4n[x]);
      else if (x < 8) read_wq(kt + 1, x - 4, wqn[x - 4]);
      else if (x < 12) sn0[x - 8] = scale_of(ws4n[x - 8], 0);
      else sn1[x - 12] = scale_of(ws4n[x - 12], 1);
      if (x < P::NLOAD) issue_one(kt + 3, x);
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(B1[j]));
    // step 3 | W step 0 of stage kt+1; its A of steps 0 and 1
    step(A3, B1, [&](int x) {
      piece(wqn[x >> 2], sn0[x >> 2], 0, x & 3, B0[x >> 2]);
      if (x < 4) read_a(kt + 1, 0, x, A0[x]);
      else if (x < 8) read_a(kt + 1, 1, x - 4, A1[x - 4]);
    });
    // the decoded W of the next step is materialised here: otherwise the
    // compiler sinks this step's decode past the loop latch, next to its use
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(B0[j]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wq[j] = wqn[j];
      sc0[j] = sn0[j];
      sc1[j] = sn1[j];
    }
  }
  // the loads of the stages past the end land before the LDS is reused
  wait_vm<0>();

  if constexpr (SPLIT) {
    // partial sums of this K slice; the reduce kernel finishes the tile
    float4* mine = part_slot(p, (int)(blockIdx.x / p.sk_tiles), tile) + wv * 64 * 64 + lane;
#pragma unroll
    for (int q = 0; q < 64; ++q) {
      const int i = q >> 4, j = (q >> 2) & 3, g = q & 3;
      mine[q * 64] = make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
    }
    return;
  }
  // bf16 output in whole 16-byte chunks: through LDS (the ring is free)
  if (staged_store_ok(p)) {
    stage_store_tile<3, 1>(p, acc, smem, m0, n0);
    return;
  }
  // epilogue: tile (i, j), lane, register e -> token row m0 + wm*128 + 32 i
  // + lane%32, feature column n0 + wn*128 + 32 j + 8 (e/4) + 4 (lane/32) + e%4
  const bool vec = out_vec_ok(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + 32 * i + r32;
    if (row >= p.M) continue;
    const float alpha = row_alpha<3>(p, row);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        emit4(p, vec, row, n0 + wn * 128 + 32 * j + 8 * g + 4 * h, alpha, acc[i][j][4 * g], acc[i][j][4 * g + 1],
              acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
  }
}

template <bool SPLIT, bool QUADS>
static hipError_t a16_set_lds() {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemm_a16_kernel<SPLIT, QUADS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, A16Pipe<QUADS>::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

template <bool QUADS>
static hipError_t launch_a16(const GemmParams& p, int dp_grid, int sk_grid, hipStream_t st) {
  const size_t lds = (size_t)A16Pipe<QUADS>::LDS;
  hipError_t e = a16_set_lds<false, QUADS>();
  if (e == hipSuccess) e = a16_set_lds<true, QUADS>();
  if (e != hipSuccess) return e;
  if (dp_grid > 0) {
    hipLaunchKernelGGL((qgemm_a16_kernel<false, QUADS>), dim3(dp_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sk_grid > 0) {
    hipLaunchKernelGGL((qgemm_a16_kernel<true, QUADS>), dim3(sk_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((qgemm_reduce_kernel<3>), dim3(p.sk_tiles * 64), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_qgemm_w4a16(const void* a, const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M, int64_t N,
                              int64_t K, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a_q = a;
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
  p.part = static_cast<float*>(ws);
  int dp_grid = 0, sk_grid = 0;
  plan_pipe(p, cu_count(), dp_grid, sk_grid, A16_BK);
  // scale quads need 16-byte aligned 16-byte runs in every scale row
  return K % 256 == 0 ? launch_a16<true>(p, dp_grid, sk_grid, st) : launch_a16<false>(p, dp_grid, sk_grid, st);
}

}  // namespace vdtq
