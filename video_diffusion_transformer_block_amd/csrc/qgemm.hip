// W4A4 (NVFP4 x NVFP4) and W4A8 (INT8 x NVFP4) GEMMs for gfx950.
//
// The operation: gist.science "6Bit-Diffusion: Inference-Time Mixed-Precision
// Quantization for Video Diffusion Models" §2.A / §3.1 (NVFP4 or INT8
// activations per block and step) and §4 (4-bit weights everywhere: W4A4
// through W4A8); youleyou.com article §四 (same operating points).
//
// Why fp16 MFMA: an NVFP4 operand is e2m1 * e4m3 per element with a scale per
// 16 elements.  CDNA4's block-scaled FP4/FP8 MFMA takes one power-of-two
// (E8M0) scale per 32 elements, so an E4M3 scale mantissa cannot ride on it,
// and e2m1 * e4m3 needs up to 6 significant bits (FP8 E4M3 holds 4).  Every
// such product, and every int8 code, is exact in fp16 (range 2^-10 .. 2688),
// so both operands are decoded to fp16 and fed to v_mfma_f32_32x32x16_f16
// with fp32 accumulation: exact products, one fp32 rounding per add, the
// tensor / token scales applied in the epilogue.  For W4A8 with unit weight
// scales the fp32 accumulator holds the integer sum exactly (< 2^24).
//
// Data flow (one workgroup = 4 wavefronts, 2 x 2; tile BM x BN, K in stages
// of 128):
//   global -> registers -> LDS   the operands stay packed (4-bit codes,
//                                E4M3 scale bytes, int8 codes): 16-byte loads,
//                                64 / 128 contiguous bytes per row and stage,
//                                written to LDS with an XOR swizzle so that
//                                the fragment reads below are conflict free;
//                                double buffered, one barrier per stage.
//   LDS -> MFMA fragments        each lane reads 32 codes of one row (one
//                                16-byte read) and the two scale bytes, and
//                                decodes them itself: the hardware fp4->f16
//                                conversion (power-of-two scale 2^8 folded in)
//                                and one packed f16 multiply by the scale
//                                whose bits are the E4M3 byte shifted into an
//                                fp16 (= scale * 2^-8); int8 -> f16 by the
//                                0x6400 bias trick.  Decoding costs about one
//                                VALU op per element per wavefront and runs
//                                beside the MFMAs.
//   K order inside a stage       lane half h and chunk c cover k = 64c + 32h
//                                .. +32; step s of a chunk takes 8 of them.
//                                A and W use the same map, so each MFMA sums
//                                matching k and the stage covers all 128.
//   tile order                   workgroups are dealt round-robin to the 8
//                                XCDs; each XCD gets a contiguous range of
//                                tile ids, walked in groups of 8 M-tiles, so
//                                the A and W stripes it needs stay in its L2.
//   work split (K % 128 == 0)    whole waves of tiles run data-parallel, one
//                                tile per workgroup; the tiles of a partial
//                                last wave are then split into K slices (one
//                                workgroup each, at most one per CU in all)
//                                when that beats the partial wave, and a
//                                reduce pass adds the fp32 slices in slice
//                                order (deterministic) and writes the output.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "qgemm_common.h"

namespace vdtq {

// --------------------------------------------------------------- decoding
// E4M3 byte pair -> fp16 pair holding scale * 2^-8 each: the 7 magnitude bits
// eeeemmm placed at fp16 bits 13..7 give exponent eeee (bias 15 instead of 7)
// and mantissa mmm, for normal and subnormal E4M3 alike.
__device__ __forceinline__ uint32_t scale_pair_bits(uint32_t s2) {
  return ((s2 & 0x7Fu) << 7) | ((s2 & 0x7F00u) << 15);
}

// 8 e2m1 codes -> 8 halves = e2m1 * 2^8 * (scale * 2^-8), exact.
__device__ __forceinline__ half8 dec_fp4x8(uint32_t w, half2v sc) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * sc;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * sc;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * sc;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * sc;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 int8 (two dwords) -> 8 halves: fp16 0x6400 | (b ^ 0x80) is 1152 + b.
__device__ __forceinline__ half8 dec_i8x8(uint32_t w0, uint32_t w1) {
  const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  half2v p0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - bias;
  half2v p1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - bias;
  half2v p2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) - bias;
  half2v p3 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) - bias;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// --------------------------------------------------------------- LDS layout
// Code rows are swizzled (fp4_quad_off / i8_quad_off); NVFP4 scales: 8 bytes
// per row and stage, unswizzled.

// One stage of packed operand rows: `rows` rows from `row0` (clamped to the
// last valid row), K columns k0 .. k0+127 (zero past K).
template <int ROWS, bool INT8>
struct StageLoader {
  static constexpr int QPR = INT8 ? 8 : 4;                 // 16-byte quads per row
  static constexpr int NQ = ROWS * QPR / GT;               // quads per thread
  static constexpr int SB = INT8 ? 0 : ROWS * 8 / GT;      // scale bytes per thread
  static constexpr int SW = SB > 0 ? (SB + 3) / 4 : 1;     // scale dwords per thread
  uint4 q[NQ];
  uint32_t s[SW];

  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int row0, int nrows,
                                       int K, int k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int G = t + GT * u;
      const int r = G / QPR, qq = G % QPR;
      const int64_t row = min(row0 + r, nrows - 1);
      // first element of this quad, and how many of its 16-element groups are in K
      const int kq = k0 + (INT8 ? 16 : 32) * qq;
      const int ngroups = INT8 ? (kq < K ? 1 : 0) : (kq + 32 <= K ? 2 : (kq < K ? 1 : 0));
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (INT8) {
        if (ngroups) v = *reinterpret_cast<const uint4*>(codes + row * K + kq);
      } else {
        const uint8_t* p = codes + row * (K / 2) + kq / 2;
        if (ngroups == 2) {
          if ((K & 31) == 0) {
            v = *reinterpret_cast<const uint4*>(p);
          } else {
            uint2 a = reinterpret_cast<const uint2*>(p)[0], b = reinterpret_cast<const uint2*>(p)[1];
            v = make_uint4(a.x, a.y, b.x, b.y);
          }
        } else if (ngroups == 1) {
          uint2 a = *reinterpret_cast<const uint2*>(p);
          v = make_uint4(a.x, a.y, 0u, 0u);
        }
      }
      q[u] = v;
    }
    if constexpr (!INT8) {
      // SB bytes per thread: thread t covers row (t*SB)/8, bytes (t*SB)%8 ..
      const int b0 = t * SB;
      const int r = b0 / 8, j0 = b0 % 8;
      const int64_t row = min(row0 + r, nrows - 1);
      const int kg = k0 / 16 + j0;                 // first group index
      const uint8_t* p = scales + row * (K / 16) + kg;
      uint32_t w[SW];
#pragma unroll
      for (int i = 0; i < SW; ++i) w[i] = 0u;
      if ((K % 128) == 0 && kg + SB <= K / 16) {
        if constexpr (SB == 8) {
          uint2 a = *reinterpret_cast<const uint2*>(p);
          w[0] = a.x;
          w[1] = a.y;
        } else {
          w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
      } else {
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (kg + i < K / 16) w[i / 4] |= (uint32_t)p[i] << (8 * (i % 4));
      }
#pragma unroll
      for (int i = 0; i < SW; ++i) s[i] = w[i];
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes, uint8_t* lds_scales) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int G = t + GT * u;
      const int r = G / QPR, qq = G % QPR;
      const int off = INT8 ? i8_quad_off(r, qq) : fp4_quad_off(r, qq);
      *reinterpret_cast<uint4*>(lds_codes + off) = q[u];
    }
    if constexpr (!INT8) {
      if constexpr (SB == 8)
        *reinterpret_cast<uint2*>(lds_scales + t * 8) = make_uint2(s[0], s[1]);
      else
        *reinterpret_cast<uint32_t*>(lds_scales + t * 4) = s[0];
    }
  }
};

template <int AFMT, int TI, int TJ>
struct Cfg {
  static constexpr int BM = 64 * TI, BN = 64 * TJ;
  static constexpr bool A8 = AFMT == 1;
  static constexpr int A_CODES = BM * (A8 ? 128 : 64);
  static constexpr int A_SC = A8 ? 0 : BM * 8;
  static constexpr int W_CODES = BN * 64;
  static constexpr int W_SC = BN * 8;
  static constexpr int STAGE = A_CODES + A_SC + W_CODES + W_SC;
};

// Tile coordinates of a data-parallel launch: XCD-contiguous id ranges.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = bid % 8, idx = bid / 8;
  const int base = nblocks / 8, rem = nblocks % 8;
  const int id = xcd * base + min(xcd, rem) + idx;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int g = id / per_group;
  const int first_m = g * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in = id - g * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

template <int AFMT, int TI, int TJ>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm_kernel(GemmParams p) {
  using C = Cfg<AFMT, TI, TJ>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  StageLoader<C::BM, C::A8> la;
  StageLoader<C::BN, false> lw;

  float16v acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint8_t* aq = static_cast<const uint8_t*>(p.a_q);
  const uint8_t* as = static_cast<const uint8_t*>(p.a_s);
  const int nk = (p.K + BK - 1) / BK;

  auto stage_ptr = [&](int buf) { return smem + buf * C::STAGE; };

  la.load(aq, as, m0, p.M, p.K, 0);
  lw.load(p.w_q, p.w_s, n0, p.N, p.K, 0);
  {
    uint8_t* s0 = stage_ptr(0);
    la.store(s0, s0 + C::A_CODES);
    lw.store(s0 + C::A_CODES + C::A_SC, s0 + C::A_CODES + C::A_SC + C::W_CODES);
  }
  __syncthreads();

  const int r32 = lane & 31, h = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      la.load(aq, as, m0, p.M, p.K, (kt + 1) * BK);
      lw.load(p.w_q, p.w_s, n0, p.N, p.K, (kt + 1) * BK);
    }
    const uint8_t* st = stage_ptr(kt & 1);
    const uint8_t* a_codes = st;
    const uint8_t* a_sc = st + C::A_CODES;
    const uint8_t* w_codes = st + C::A_CODES + C::A_SC;
    const uint8_t* w_sc = w_codes + C::W_CODES;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qd = 2 * c + h;
      uint4 araw[TI][C::A8 ? 2 : 1];
      uint32_t asc[TI];
      uint4 wraw[TJ];
      uint32_t wsc[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wm * 32 * TI + 32 * i + r32;
        if (C::A8) {
          araw[i][0] = *reinterpret_cast<const uint4*>(a_codes + i8_quad_off(row, 2 * qd));
          araw[i][C::A8 ? 1 : 0] = *reinterpret_cast<const uint4*>(a_codes + i8_quad_off(row, 2 * qd + 1));
          asc[i] = 0u;
        } else {
          araw[i][0] = *reinterpret_cast<const uint4*>(a_codes + fp4_quad_off(row, qd));
          asc[i] = scale_pair_bits(*reinterpret_cast<const uint16_t*>(a_sc + row * 8 + 4 * c + 2 * h));
        }
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wn * 32 * TJ + 32 * j + r32;
        wraw[j] = *reinterpret_cast<const uint4*>(w_codes + fp4_quad_off(row, qd));
        wsc[j] = scale_pair_bits(*reinterpret_cast<const uint16_t*>(w_sc + row * 8 + 4 * c + 2 * h));
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8 af[TI], bf[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          if (C::A8) {
            const uint4& v = araw[i][s >> 1];
            af[i] = (s & 1) ? dec_i8x8(v.z, v.w) : dec_i8x8(v.x, v.y);
          } else {
            const half2v sp = __builtin_bit_cast(half2v, asc[i]);
            const half2v sc = (s < 2) ? half2v{sp[0], sp[0]} : half2v{sp[1], sp[1]};
            const uint32_t w = s == 0 ? araw[i][0].x : s == 1 ? araw[i][0].y : s == 2 ? araw[i][0].z : araw[i][0].w;
            af[i] = dec_fp4x8(w, sc);
          }
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const half2v sp = __builtin_bit_cast(half2v, wsc[j]);
          const half2v sc = (s < 2) ? half2v{sp[0], sp[0]} : half2v{sp[1], sp[1]};
          const uint32_t w = s == 0 ? wraw[j].x : s == 1 ? wraw[j].y : s == 2 ? wraw[j].z : wraw[j].w;
          bf[j] = dec_fp4x8(w, sc);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) {
      uint8_t* sn = stage_ptr((kt + 1) & 1);
      la.store(sn, sn + C::A_CODES);
      lw.store(sn + C::A_CODES + C::A_SC, sn + C::A_CODES + C::A_SC + C::W_CODES);
    }
    __syncthreads();
  }

  // epilogue: MFMA tile (i, j), lane, register e -> row 8*(e/4) + 4*(lane/32)
  // + e%4, col lane%32.  Decoded operands carry no extra factor (the 2^8 of
  // the fp4 conversion cancels the 2^-8 of the scale bits).
  const float gsw = p.w_ts[1];
  const float alpha_t = (AFMT == 0) ? p.a_ts[1] * gsw : 0.0f;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + wm * 32 * TI + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
      if (row >= p.M) continue;
      const float alpha = (AFMT == 0) ? alpha_t : static_cast<const float*>(p.a_s)[row] * gsw;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn * 32 * TJ + 32 * j + r32;
        if (col >= p.N) continue;
        float v = acc[i][j][e] * alpha;
        if (p.bias) v = v + p.bias[col];
        if (p.out_f32)
          static_cast<float*>(p.y)[(int64_t)row * p.ldy + col] = v;
        else
          static_cast<uint16_t*>(p.y)[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

// =============================================================== pipelined
// Fast path for K % 128 == 0: the same 256 x 256 tile and fragment decode,
// with
//   * direct-to-LDS loads (global_load_lds: each lane names the global 16-byte
//     quad that lands in its LDS slot, which applies the XOR swizzle) into a
//     3-deep ring of stages, issued two stages ahead;
//   * one barrier per stage, placed mid-stage: each wave first waits for its
//     own loads of the next stage (vmcnt) and for its LDS reads of the current
//     one (lgkmcnt), so after the barrier the next stage is complete and the
//     current buffer is free for the stage three ahead;
//   * a step-level software pipeline scheduled by hand: each of the 16
//     MFMAs of step s is followed by a quarter fragment of the decode of
//     step s+1 (two conversions, two multiplies) and at most one LDS read
//     or scale operation, held together by sched_barrier, so the VALU work
//     runs under the MFMAs instead of in bursts between them.
// PAIRS (K % 256 == 0): the E4M3 scales of two consecutive stages (16
// contiguous bytes per row) arrive in one 16-byte load per row, into a
// double-buffered pair region after the ring, instead of two 4-byte loads
// per row and stage.
template <int AFMT, bool PAIRS>
struct Pipe {
  static constexpr bool A8 = AFMT == 1;
  static constexpr int A_CODES = 256 * (A8 ? 128 : 64);
  static constexpr int A_SC = (A8 || PAIRS) ? 0 : 256 * 8;
  static constexpr int W_CODES = 256 * 64;
  static constexpr int W_SC = PAIRS ? 0 : 256 * 8;
  static constexpr int STAGE = A_CODES + A_SC + W_CODES + W_SC;
  static constexpr int NS = 3;
  static constexpr int NA = A8 ? 8 : 4;                 // A code loads per wave and stage (1 KB each)
  static constexpr int NAS = (A8 || PAIRS) ? 0 : 2;     // A scale loads per wave and stage (256 B each)
  static constexpr int NW = 4;
  static constexpr int NWS = PAIRS ? 0 : 2;
  static constexpr int LPS = NA + NAS + NW + NWS;       // loads per wave and stage (pairs apart)
  static constexpr int PAIR_A = (PAIRS && !A8) ? 256 * 16 : 0;
  static constexpr int PAIR_W = PAIRS ? 256 * 16 : 0;
  static constexpr int PAIR_SLOT = PAIR_A + PAIR_W;
  static constexpr int PAIR_BASE = NS * STAGE;
  static constexpr int NPAIR = (PAIR_A ? 1 : 0) + (PAIR_W ? 1 : 0);   // pair loads per wave
  // a 1 KB LDS landing area per wave for the loads of stages past the last:
  // every stage issues the same loads (no branch), those past the end
  // read valid addresses and land here
  static constexpr int DUMMY = NS * STAGE + 2 * PAIR_SLOT;
  static constexpr int NDMA = LPS + NPAIR;             // loads per wave and stage, scale pair included
  static constexpr int LDS = DUMMY + 4 * 1024;
};

// per-chunk raw operands of one lane: codes for its 4 A and 4 W sub-blocks
template <bool A8>
struct Raw {
  uint4 a[4][A8 ? 2 : 1];
  uint4 w[4];
};

// SPLIT = false: one whole tile per workgroup, tiles sk_tiles .. tiles-1
// dealt in XCD-contiguous ranges (hardware dispatch balances the CUs).
// SPLIT = true: one K slice of one of the tiles 0 .. sk_tiles-1 per
// workgroup; the fp32 partial sums go to the workspace and qgemm_reduce_kernel
// adds the slices and writes the output.
template <int AFMT, bool SPLIT, bool PAIRS>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm_pipe_kernel(GemmParams p) {
  using P = Pipe<AFMT, PAIRS>;
  constexpr bool A8 = P::A8;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = p.K;
  const int nk = p.nk;

  const uint8_t* aq = static_cast<const uint8_t*>(p.a_q);
  const uint8_t* as = static_cast<const uint8_t*>(p.a_s);

  // ---- per-lane byte offsets of the DMA sources at k0 = 0 for the current
  // tile (32-bit: every operand matrix is below 4 GB, checked on the host)
  uint32_t offA[P::NA], offAS[P::NAS > 0 ? P::NAS : 1], offW[P::NW], offWS[P::NWS > 0 ? P::NWS : 1];
  uint32_t offAP = 0, offWP = 0;   // scale pairs: row wv*64 + lane
  int m0 = 0, n0 = 0;
  auto set_tile = [&](int tile) {
  int tm, tn;
  tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
  m0 = tm * 256;
  n0 = tn * 256;
#pragma unroll
  for (int u = 0; u < P::NA; ++u) {
    if (A8) {
      const int r = (wv * P::NA + u) * 8 + (lane >> 3);
      const int q = (lane & 7) ^ (r & 7);
      offA[u] = (uint32_t)min(m0 + r, p.M - 1) * (uint32_t)K + 16u * q;
    } else {
      const int r = (wv * P::NA + u) * 16 + (lane >> 2);
      const int q = (lane & 3) ^ ((r >> 1) & 3);
      offA[u] = (uint32_t)min(m0 + r, p.M - 1) * (uint32_t)(K / 2) + 16u * q;
    }
  }
#pragma unroll
  for (int u = 0; u < P::NAS; ++u) {
    const int r = (wv * P::NAS + u) * 32 + (lane >> 1);
    offAS[u] = (uint32_t)min(m0 + r, p.M - 1) * (uint32_t)(K / 16) + 4u * (lane & 1);
  }
#pragma unroll
  for (int u = 0; u < P::NW; ++u) {
    const int r = (wv * P::NW + u) * 16 + (lane >> 2);
    const int q = (lane & 3) ^ ((r >> 1) & 3);
    offW[u] = (uint32_t)min(n0 + r, p.N - 1) * (uint32_t)(K / 2) + 16u * q;
  }
#pragma unroll
  for (int u = 0; u < P::NWS; ++u) {
    const int r = (wv * P::NWS + u) * 32 + (lane >> 1);
    offWS[u] = (uint32_t)min(n0 + r, p.N - 1) * (uint32_t)(K / 16) + 4u * (lane & 1);
  }
  if (PAIRS) {
    offAP = (uint32_t)min(m0 + wv * 64 + lane, p.M - 1) * (uint32_t)(K / 16);
    offWP = (uint32_t)min(n0 + wv * 64 + lane, p.N - 1) * (uint32_t)(K / 16);
  }
  };

  // LDS byte address of smem and of this wave's regions (wave-uniform)
  const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t*)smem;
  const uint32_t wvu = __builtin_amdgcn_readfirstlane(wv);
  // ring slot of stage kt: counted from the first stage of the segment
  int kbase = 0;
  int tile, kb, ke;
  auto ring = [&](int kt) { return (kt - kbase) % P::NS; };
  // Load u (0 .. NDMA-1) of stage kt, branch-free: a stage past the last
  // reads stage ke-1's addresses into this wave's landing area, and the
  // scale-pair loads go out every stage, to the landing area unless the
  // stage is even or the segment's first (the pair (kt & ~1, kt | 1)).
  // Such a load reads the same 16 bytes in every lane (offset 0 from the
  // stage's base), one memory request instead of one per row.
  const uint32_t dummy = lds0 + P::DUMMY + wvu * 1024;
  // (the destination is chosen by masks, not branches: the step stays one
  // basic block, so its schedule holds)
  auto pick = [&](uint32_t m, uint32_t target) { return dummy + ((target - dummy) & m); };
  auto issue_one = [&](int kt, int u) {
    const uint32_t live = 0u - (uint32_t)(kt < ke);
    const int ks = min(kt, ke - 1);
    const uint32_t st = lds0 + (uint32_t)ring(kt) * P::STAGE;
    const int k0 = ks * BK;
    if (u < P::NA) {
      dma16(aq + (A8 ? k0 : k0 / 2), offA[u] & live, pick(live, st + (wvu * P::NA + u) * 1024));
    } else if (u < P::NA + P::NAS) {
      const int v = u - P::NA;
      dma4(as + k0 / 16, offAS[v] & live, pick(live, st + P::A_CODES + (wvu * P::NAS + v) * 256));
    } else if (u < P::NA + P::NAS + P::NW) {
      const int v = u - P::NA - P::NAS;
      dma16(p.w_q + k0 / 2, offW[v] & live, pick(live, st + P::A_CODES + P::A_SC + (wvu * P::NW + v) * 1024));
    } else if (u < P::LPS) {
      const int v = u - P::NA - P::NAS - P::NW;
      dma4(p.w_s + k0 / 16, offWS[v] & live, pick(live, st + P::A_CODES + P::A_SC + P::W_CODES + (wvu * P::NWS + v) * 256));
    } else if (PAIRS) {
      const uint32_t real = live & (0u - (uint32_t)(((kt & 1) == 0) | (kt == kbase)));
      const int pr = ks >> 1;
      const uint32_t ps = lds0 + P::PAIR_BASE + (uint32_t)(pr & 1) * P::PAIR_SLOT + wvu * 64 * 16;
      if (P::PAIR_A && u == P::LPS) dma16(as + 16 * pr, offAP & real, pick(real, ps));
      else dma16(p.w_s + 16 * pr, offWP & real, pick(real, ps + P::PAIR_A));
    }
  };
  auto issue_stage = [&](int kt) {
#pragma unroll
    for (int u = 0; u < P::NDMA; ++u) issue_one(kt, u);
  };

  // ---- LDS read offsets of this lane's fragments (within a stage)
  const int r32 = lane & 31, h = lane >> 5;
  auto read_codes = [&](int kt, int c, Raw<A8>& R) {
    const uint8_t* st = smem + ring(kt) * P::STAGE;
    const int qd = 2 * c + h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + r32;
      if (A8) {
        R.a[i][0] = *reinterpret_cast<const uint4*>(st + i8_quad_off(row, 2 * qd));
        R.a[i][A8 ? 1 : 0] = *reinterpret_cast<const uint4*>(st + i8_quad_off(row, 2 * qd + 1));
      } else {
        R.a[i][0] = *reinterpret_cast<const uint4*>(st + fp4_quad_off(row, qd));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + 32 * j + r32;
      R.w[j] = *reinterpret_cast<const uint4*>(st + P::A_CODES + P::A_SC + fp4_quad_off(row, qd));
    }
  };
  // the 8 scale bytes (groups of both chunks) of each of this lane's rows
  auto read_scales = [&](int kt, uint2 (&sa)[4], uint2 (&sw)[4]) {
    if (PAIRS) {
      const uint8_t* ps = smem + P::PAIR_BASE + ((kt >> 1) & 1) * P::PAIR_SLOT + (kt & 1) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!A8) sa[i] = *reinterpret_cast<const uint2*>(ps + (wm * 128 + 32 * i + r32) * 16);
        else sa[i] = make_uint2(0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sw[j] = *reinterpret_cast<const uint2*>(ps + P::PAIR_A + (wn * 128 + 32 * j + r32) * 16);
      return;
    }
    const uint8_t* st = smem + ring(kt) * P::STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!A8) sa[i] = *reinterpret_cast<const uint2*>(st + P::A_CODES + (wm * 128 + 32 * i + r32) * 8);
      else sa[i] = make_uint2(0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sw[j] = *reinterpret_cast<const uint2*>(st + P::A_CODES + P::A_SC + P::W_CODES + (wn * 128 + 32 * j + r32) * 8);
  };
  // scale pair of chunk c for this lane half: groups 4c + 2h, 4c + 2h + 1.
  // One byte permute moves bytes 2h and 2h + 1 of the chunk's dword into
  // bytes 0 and 2 (zeros elsewhere) and one shift by 7 makes each 16-bit
  // half the fp16 scale * 2^-8 of scale_pair_bits, for scale bytes with the
  // sign bit clear (every scale the quantizer writes is >= 0).
  const uint32_t ssel = 0x0C000C00u | ((2u * (uint32_t)h + 1u) << 16) | (2u * (uint32_t)h);
  auto scale_of = [&](const uint2& s8, int c) { return __builtin_amdgcn_perm(0u, c ? s8.y : s8.x, ssel) << 7; };

  auto decode = [&](const Raw<A8>& R, const uint2 (&sa)[4], const uint2 (&sw)[4], int c, int s,
                    half8 (&af)[4], half8 (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (A8) {
        const uint4& v = R.a[i][s >> 1];
        af[i] = (s & 1) ? dec_i8x8(v.z, v.w) : dec_i8x8(v.x, v.y);
      } else {
        const half2v sp = __builtin_bit_cast(half2v, scale_of(sa[i], c));
        const half2v sc = (s < 2) ? half2v{sp[0], sp[0]} : half2v{sp[1], sp[1]};
        const uint4& v = R.a[i][0];
        af[i] = dec_fp4x8(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w, sc);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2v sp = __builtin_bit_cast(half2v, scale_of(sw[j], c));
      const half2v sc = (s < 2) ? half2v{sp[0], sp[0]} : half2v{sp[1], sp[1]};
      const uint4& v = R.w[j];
      bf[j] = dec_fp4x8(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w, sc);
    }
  };

  float16v acc[4][4];
  if constexpr (SPLIT) {
    tile = (int)(blockIdx.x % p.sk_tiles);
    const int sl = (int)(blockIdx.x / p.sk_tiles);
    kb = sl * p.slice_nk;
    ke = min(nk, kb + p.slice_nk);
  } else {
    tile = p.sk_tiles + xcd_range_id(blockIdx.x, gridDim.x);
    kb = 0;
    ke = nk;
  }
  set_tile(tile);
  kbase = kb;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // ---- prologue: stages kb..kb+2 in flight (those past the end land in
  // the landing area), wait for stage kb
  issue_stage(kb);
  issue_stage(kb + 1);
  issue_stage(kb + 2);
  wait_vm<2 * P::NDMA>();
  wait_lgkm_barrier();

  Raw<A8> R0, R1;
  uint2 sa[4], sw[4], na[4], nw[4];
  half8 fa[4], fb[4], ga[4], gb[4];
  read_codes(kb, 0, R0);
  read_scales(kb, sa, sw);
  decode(R0, sa, sw, 0, 0, fa, fb);

  // ---- the main loop, scheduled by hand.  A step is 16 MFMAs; after MFMA
  // x comes piece x of the decode of the next step's operands (fragment
  // x / 2 of 4 A + 4 W, elements 4 (x % 2) .. +3: two conversions and two
  // multiplies) and at most one LDS read or scale operation, and a
  // sched_barrier keeps each MFMA with its slot.  One wave runs per SIMD,
  // so the matrix core stays busy only if no run of VALU work outlasts an
  // MFMA and no MFMAs are issued back to back.
  //
  // Scale registers of a chunk: per fragment f (A 0-3, W 4-7) lo = the fp16
  // scale pair bits (the group of steps 0-1 in the low half) and hi = the
  // group of steps 2-3 moved to the low half.
  uint32_t S0lo[8], S0hi[8], S1lo[8], S1hi[8];
  auto scale_lo = [&](const uint2 (&xa)[4], const uint2 (&xw)[4], int c, int f, uint32_t (&lo)[8]) {
    if (f < 4) {
      if (!A8) lo[f] = scale_of(xa[f], c);
    } else {
      lo[f] = scale_of(xw[f - 4], c);
    }
  };
  auto scale_hi = [&](int f, const uint32_t (&lo)[8], uint32_t (&hi)[8]) {
    if (f >= 4 || !A8) hi[f] = lo[f] >> 16;
  };
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    scale_lo(sa, sw, 0, f, S0lo);
    scale_hi(f, S0lo, S0hi);
  }
  // piece x of the decode of step s of a chunk (codes R, scales lo / hi)
  auto piece = [&](const Raw<A8>& R, int s, const uint32_t (&lo)[8], const uint32_t (&hi)[8], half8 (&NA)[4],
                   half8 (&NB)[4], int x) {
    const int f = x >> 1, h2 = x & 1;
    if (A8 && f < 4) {
      const uint4& v = R.a[f][s >> 1];
      const uint32_t w = h2 ? ((s & 1) ? v.w : v.y) : ((s & 1) ? v.z : v.x);
      const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
      const uint32_t x0 = w ^ 0x80808080u;
      const half2v p0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - bias;
      const half2v p1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - bias;
      NA[f][4 * h2 + 0] = p0[0]; NA[f][4 * h2 + 1] = p0[1];
      NA[f][4 * h2 + 2] = p1[0]; NA[f][4 * h2 + 3] = p1[1];
    } else {
      const half2v sp = __builtin_bit_cast(half2v, s < 2 ? lo[f] : hi[f]);
      const half2v sc = {sp[0], sp[0]};
      const uint4& v = f < 4 ? R.a[f][0] : R.w[f - 4];
      const uint32_t w = s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
      // (the byte index of the conversion is an immediate)
      const half2v p0 = (h2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0)) * sc;
      const half2v p1 = (h2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1)) * sc;
      half8& o = f < 4 ? NA[f] : NB[f - 4];
      o[4 * h2 + 0] = p0[0]; o[4 * h2 + 1] = p0[1];
      o[4 * h2 + 2] = p1[0]; o[4 * h2 + 3] = p1[1];
    }
  };
  // one LDS read of chunk c's codes of stage kt: A fragment reads first
  // (INT8: two per fragment), then the four W fragments
  constexpr int NAR = A8 ? 8 : 4;
  auto read_code = [&](int kt, int c, Raw<A8>& R, int r) {
    const uint8_t* st = smem + ring(kt) * P::STAGE;
    const int qd = 2 * c + h;
    if (r < NAR) {
      if (A8) {
        const int i = r >> 1, half = r & 1;
        R.a[i][half] = *reinterpret_cast<const uint4*>(st + i8_quad_off(wm * 128 + 32 * i + r32, 2 * qd + half));
      } else {
        R.a[r][0] = *reinterpret_cast<const uint4*>(st + fp4_quad_off(wm * 128 + 32 * r + r32, qd));
      }
    } else {
      const int j = r - NAR;
      R.w[j] = *reinterpret_cast<const uint4*>(st + P::A_CODES + P::A_SC + fp4_quad_off(wn * 128 + 32 * j + r32, qd));
    }
  };
  // one LDS read of the 8 scale bytes of fragment f (A 0-3, W 4-7) of stage kt
  auto read_scale = [&](int kt, int f, uint2 (&xa)[4], uint2 (&xw)[4]) {
    if (f < 4 && A8) {
      xa[f] = make_uint2(0u, 0u);
      return;
    }
    const int row = (f < 4 ? wm : wn) * 128 + 32 * (f & 3) + r32;
    const uint8_t* src;
    if (PAIRS) {
      const uint8_t* ps = smem + P::PAIR_BASE + ((kt >> 1) & 1) * P::PAIR_SLOT + (kt & 1) * 8;
      src = f < 4 ? ps + row * 16 : ps + P::PAIR_A + row * 16;
    } else {
      const uint8_t* st = smem + ring(kt) * P::STAGE;
      src = f < 4 ? st + P::A_CODES + row * 8 : st + P::A_CODES + P::A_SC + P::W_CODES + row * 8;
    }
    (f < 4 ? xa[f] : xw[f - 4]) = *reinterpret_cast<const uint2*>(src);
  };
  auto step = [&](const half8 (&CA)[4], const half8 (&CB)[4], auto&& work) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(CB[x & 3], CA[x >> 2], acc[x >> 2][x & 3], 0, 0, 0);
      work(x);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Every step has the same shape; past the last stage the reads of the
  // "next" stage hit a stale ring slot and the extra decode is discarded.
  for (int kt = kb; kt < ke; ++kt) {
    // step 0 | decode chunk 0 step 1
    step(fa, fb, [&](int x) { piece(R0, 1, S0lo, S0hi, ga, gb, x); });
    // step 1 | decode chunk 0 step 2; read chunk 1 codes
    step(ga, gb, [&](int x) {
      piece(R0, 2, S0lo, S0hi, fa, fb, x);
      if (x < NAR + 4) read_code(kt, 1, R1, x);
    });
    // step 2 | decode chunk 0 step 3; chunk 1 scale registers
    step(fa, fb, [&](int x) {
      piece(R0, 3, S0lo, S0hi, ga, gb, x);
      if (x < 8) scale_lo(sa, sw, 1, x, S1lo);
      else scale_hi(x - 8, S1lo, S1hi);
    });
    // step 3 | decode chunk 1 step 0
    step(ga, gb, [&](int x) { piece(R1, 0, S1lo, S1hi, fa, fb, x); });
    // mid-stage barrier: next stage complete (only stage kt+2's loads may
    // still be in flight), this buffer free
    wait_vm<P::NDMA>();
    wait_lgkm_barrier();
    // step 4 | decode chunk 1 step 1; read stage kt+1's scales; issue the
    // loads of stage kt+3 into the buffer just freed
    step(fa, fb, [&](int x) {
      piece(R1, 1, S1lo, S1hi, ga, gb, x);
      if (x < 8) read_scale(kt + 1, x, na, nw);
      if (x < P::NDMA) issue_one(kt + 3, x);
    });
    // step 5 | decode chunk 1 step 2; read stage kt+1's chunk 0 codes
    step(ga, gb, [&](int x) {
      piece(R1, 2, S1lo, S1hi, fa, fb, x);
      if (x < NAR + 4) read_code(kt + 1, 0, R0, x);
    });
    // step 6 | decode chunk 1 step 3; stage kt+1's chunk 0 scale registers
    step(fa, fb, [&](int x) {
      piece(R1, 3, S1lo, S1hi, ga, gb, x);
      if (x < 8) scale_lo(na, nw, 0, x, S0lo);
      else scale_hi(x - 8, S0lo, S0hi);
    });
    // step 7 | decode step 0 of stage kt+1
#pragma unroll
    for (int i = 0; i < 4; ++i) { sa[i] = na[i]; sw[i] = nw[i]; }
    step(ga, gb, [&](int x) { piece(R0, 0, S0lo, S0hi, fa, fb, x); });
  }
  // the loads of the stages past the end must land before the workgroup's
  // LDS is released or reused
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
    stage_store_tile<AFMT, (P::LDS >= 4 * 32768) ? 1 : 2>(p, acc, smem, m0, n0);
    return;
  }
  // epilogue: tile (i, j), lane, register e -> token row m0 + wm*128 + 32 i
  // + lane%32, feature column n0 + wn*128 + 32 j + 8 (e/4) + 4 (lane/32) + e%4
  const bool vec = out_vec_ok(p);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + 32 * i + r32;
    if (row >= p.M) continue;
    const float alpha = row_alpha<AFMT>(p, row);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        emit4(p, vec, row, n0 + wn * 128 + 32 * j + 8 * g + 4 * h, alpha, acc[i][j][4 * g], acc[i][j][4 * g + 1],
              acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
  }
}

template <int AFMT, bool SPLIT, bool PAIRS>
static hipError_t set_lds_attr() {
  using P = Pipe<AFMT, PAIRS>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemm_pipe_kernel<AFMT, SPLIT, PAIRS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, P::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

template <int AFMT, bool PAIRS>
static hipError_t launch_pipe(GemmParams p, int dp_grid, int sk_grid, hipStream_t st) {
  using P = Pipe<AFMT, PAIRS>;
  const size_t lds = (size_t)P::LDS;
  hipError_t e = set_lds_attr<AFMT, false, PAIRS>();
  if (e == hipSuccess) e = set_lds_attr<AFMT, true, PAIRS>();
  if (e != hipSuccess) return e;
  if (dp_grid > 0) {
    hipLaunchKernelGGL((qgemm_pipe_kernel<AFMT, false, PAIRS>), dim3(dp_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sk_grid > 0) {
    hipLaunchKernelGGL((qgemm_pipe_kernel<AFMT, true, PAIRS>), dim3(sk_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((qgemm_reduce_kernel<AFMT>), dim3(p.sk_tiles * 64), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

template <int AFMT, int TI, int TJ>
static hipError_t launch_cfg(GemmParams p, hipStream_t st) {
  using C = Cfg<AFMT, TI, TJ>;
  p.tiles_m = (p.M + C::BM - 1) / C::BM;
  p.tiles_n = (p.N + C::BN - 1) / C::BN;
  const int nblocks = p.tiles_m * p.tiles_n;
  const size_t lds = 2 * (size_t)C::STAGE;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemm_kernel<AFMT, TI, TJ>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((qgemm_kernel<AFMT, TI, TJ>), dim3(nblocks), dim3(GT), lds, st, p);
  return hipGetLastError();
}

size_t qgemm_workspace_bytes(int64_t M, int64_t N) {
  if (M <= 0 || N <= 0) return 0;
  // at most one K slice per CU (kGemmMaxGrid) is in flight
  return (size_t)kGemmMaxGrid * 256 * 256 * sizeof(float);
}

hipError_t launch_qgemm(int afmt, const void* a_q, const void* a_s, const float* a_ts,
                        const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                        const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                        int64_t N, int64_t K, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_ts = a_ts;
  p.w_q = w_q; p.w_s = w_s; p.w_ts = w_ts;
  p.bias = bias; p.y = y; p.ldy = ldy;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.out_f32 = out_dtype == 1;
  p.part = static_cast<float*>(ws);
  // The pipelined kernel needs whole 128-wide K stages and 32-bit byte
  // offsets into every operand matrix.
  const bool fast = (K % BK) == 0 && (afmt == 1 ? M * K : M * K / 2) < (int64_t(1) << 32) &&
                    N * K / 2 < (int64_t(1) << 32);
  if (fast) {
    int dp_grid = 0, sk_grid = 0;
    plan_pipe(p, cu_count(), dp_grid, sk_grid);
    // whole scale pairs (K % 256 == 0) and 16-byte aligned scale rows
    const bool pairs = (p.nk % 2) == 0 && (reinterpret_cast<uintptr_t>(w_s) & 15u) == 0 &&
                       (afmt == 1 || (reinterpret_cast<uintptr_t>(a_s) & 15u) == 0);
    if (afmt == 0) return pairs ? launch_pipe<0, true>(p, dp_grid, sk_grid, st) : launch_pipe<0, false>(p, dp_grid, sk_grid, st);
    return pairs ? launch_pipe<1, true>(p, dp_grid, sk_grid, st) : launch_pipe<1, false>(p, dp_grid, sk_grid, st);
  }
  if (afmt == 0) return launch_cfg<0, 4, 4>(p, st);
  return launch_cfg<1, 4, 4>(p, st);
}

}  // namespace vdtq
