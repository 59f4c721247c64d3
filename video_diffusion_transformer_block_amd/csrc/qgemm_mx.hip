// MX-native GEMM for gfx950: MXFP4 or MXFP8 activations x MXFP4 weights on
// the block-scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4.
//
// The operation: gist.science "6Bit-Diffusion: Inference-Time Mixed-Precision
// Quantization for Video Diffusion Models" §2.A / §3.1 and §4 (4-bit weights
// everywhere; 4- or 8-bit activations chosen per block and step), with the
// operands in the OCP Microscaling (MX v1.0) formats instead of NVFP4 /
// INT8: the pages name NVFP4 as a Blackwell format, and CDNA4's matrix
// cores read E2M1 / E4M3 elements with one E8M0 scale per 32 elements
// directly, so the operands go from LDS to the matrix core undecoded.
//
// Y = sum over 32-element blocks of 2^(sa - 127) * 2^(sw - 127) *
//     (A codes . W codes) + bias; no tensor scale.
//
// Operand layout of the instruction (32 rows x 64 K per operand, checked on
// the hardware): lane l holds row l % 32.  E2M1: the 32 elements k = 32
// (l / 32) .. +31, packed as in memory (16 bytes).  E4M3: bytes 0-15 hold
// k = 16 (l / 32) .. +15 and bytes 16-31 hold k = 32 + 16 (l / 32) .. +15.
// The E8M0 scale of row r and block b (k = 32 b .. +31) is read from lane
// r + 32 b, the byte chosen by op_sel.  Output register e of lane l is
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
//
// Data flow (the shape of the NVFP4 / INT8 kernel without its decode):
//   * 256 x 256 output tile per workgroup, 4 wavefronts of 128 x 128 (4 x 4
//     instructions of 32 x 32), stages of 128 K;
//   * direct-to-LDS loads (each lane names the global 16-byte quad that
//     lands in its LDS slot, which applies the XOR swizzle) into a ring of
//     NS stages, all NS in flight; one barrier per stage, after the first of
//     its two 64-K steps, frees the stage for the load NS stages ahead;
//   * per step one 16-byte LDS read per fragment (two for E4M3) and 16
//     matrix instructions; the reads of the next step run under them;
//   * scales: one dword per row and stage (4 blocks); a lane shifts its
//     row's dword by 8 (l / 32) bits so that op_sel 0 / 2 picks its block of
//     step 0 / 1.  With K % 512 == 0 (QUADS) a row's dwords of four
//     consecutive stages are one 16-byte load per operand row, issued with
//     every fourth stage into a double-buffered region after the ring (a
//     scale load touches one row per lane, so per-stage 4-byte loads cost
//     as many memory requests as the operand codes for a sixteenth of their
//     bytes); each lane reads its rows' 16 bytes every stage and picks the
//     stage's dword.  Otherwise each stage carries its own scale dwords;
//   * the tile order, the split of a partial last wave into K slices, the
//     reduce pass and the bf16 epilogue through LDS are those of the NVFP4 /
//     INT8 kernel (qgemm_common.h).
//   * quantizing epilogue (qgemm_mx_quant; FFN-up feeding FFN-down): the
//     finished bf16 tile goes through LDS as in the bf16 epilogue, then each
//     lane takes whole 64-element row chunks of it: GELU from the device's
//     table, which the workgroup copies into LDS while its first loads are
//     in flight, the 64-point
//     Hadamard butterflies, the MX encoding; only codes and scales reach
//     HBM.  Tiles are never split along K on this path (the epilogue needs
//     the whole sum).
#include <type_traits>

#include "device_common.h"
#include "hadamard_common.h"
#include "launch.h"
#include "lds_dma.h"
#include "qgemm_common.h"

namespace vdtq {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));

// instruction operand formats (cbsz / blgp)
constexpr int kMfmaFp8 = 0;
constexpr int kMfmaFp4 = 4;

template <bool A8, bool QUADS>
struct MxPipe {
  static constexpr int A_CODES = 256 * (A8 ? 128 : 64);   // code bytes per stage
  static constexpr int W_CODES = 256 * 64;
  static constexpr int A_SC = 256 * 4;                     // 4 E8M0 bytes per row and stage
  static constexpr int W_SC = 256 * 4;
  static constexpr int STAGE = A_CODES + W_CODES + (QUADS ? 0 : A_SC + W_SC);
  // ring depth: a third E4M3 stage measured no faster than two
  static constexpr int NS = A8 ? (QUADS ? 2 : 3) : 4;
  static constexpr int NA = A_CODES / (4 * 1024);           // 16-byte loads per wave and stage
  static constexpr int NW = W_CODES / (4 * 1024);
  // loads per stage as the waits count them: with QUADS the scale loads of
  // every fourth stage are left out, so a wait for "n stages in flight"
  // waits for at most n * LPS loads and is, if anything, stricter
  static constexpr int LPS = NA + NW + (QUADS ? 0 : 2);
  static constexpr int SQ = NS * STAGE;                      // scale quads: 2 buffers x (A, W) x 256 rows x 16 B
  static constexpr int LDS = SQ + (QUADS ? 2 * 2 * 256 * 16 : 0);
  // the quantizing epilogue stages 128 KB; its GELU table lies past that
  static constexpr int GTAB = LDS > 131072 ? LDS : 131072;
};

// s_waitcnt vmcnt(n * LPS) for n whole stages left in flight (n <= 3)
template <int LPS>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 3) wait_vm<3 * LPS>();
  else if (n == 2) wait_vm<2 * LPS>();
  else if (n == 1) wait_vm<LPS>();
  else wait_vm<0>();
}

template <bool A8>
struct MxFrag {
  std::conditional_t<A8, int8v, int4v> a[4];   // E4M3: 32 bytes per lane; E2M1: 16
  int4v w[4];
};

// an operand register block of the instruction (E2M1 uses the low 4 dwords)
__device__ __forceinline__ int8v mx_operand(const int8v& v) { return v; }
__device__ __forceinline__ int8v mx_operand(const int4v& v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// Quantizing epilogue of a 256 x 256 tile: bf16(acc + bias) written to LDS
// exactly as stage_store_tile does (the same values the bf16 output would
// hold), then per lane 4 row chunks of 64 elements: optional GELU (table),
// Hadamard butterflies h = 1 .. 32, MX encoding (E2M1 or E4M3 with E8M0
// per 32).  Lanes 2r and 2r + 1 take the two chunks of one row, so their
// code stores are contiguous.  The caller has finished every LDS read of
// the ring; gtab is filled and a barrier has passed since.
template <bool FP8OUT>
__device__ __forceinline__ void quant_store_tile(const GemmParams& p, const float16v (&acc)[4][4], uint8_t* smem,
                                                 const uint16_t* gtab, int m0, int n0) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1, r32 = lane & 31, h = lane >> 5;
  uint8_t* reg = smem + wv * 32768;
  float4 bias[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bias[j][g] = p.bias ? *reinterpret_cast<const float4*>(p.bias + min(n0 + wn * 128 + 32 * j + 8 * g + 4 * h, p.N - 4))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();   // every wave is past its last read of the ring
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = 32 * i + r32;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 b = bias[j][g];
        const float v0 = acc[i][j][4 * g] * 1.0f + b.x, v1 = acc[i][j][4 * g + 1] * 1.0f + b.y;
        const float v2 = acc[i][j][4 * g + 2] * 1.0f + b.z, v3 = acc[i][j][4 * g + 3] * 1.0f + b.w;
        const int c = (4 * j + g) ^ (lrow & 15);
        *reinterpret_cast<uint2*>(reg + lrow * 256 + 16 * c + 8 * h) = make_uint2(bf16_pair(v0, v1), bf16_pair(v2, v3));
      }
  }
  // the same wave reads back what it wrote (LDS operations of a wave run in order)
  const bool gelu = (p.qflags & 4u) != 0;
  const int half = lane & 1;
#pragma unroll 2
  for (int it = 0; it < 4; ++it) {
    const int lrow = 32 * it + (lane >> 1);
    float v[64];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int c = 8 * half + jj;
      const uint4 w = *reinterpret_cast<const uint4*>(reg + lrow * 256 + 16 * (c ^ (lrow & 15)));
      const uint32_t in[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = gelu ? gelu_word(in[q], gtab) : in[q];
        v[8 * jj + 2 * q] = __uint_as_float(x << 16);
        v[8 * jj + 2 * q + 1] = __uint_as_float(x & 0xFFFF0000u);
      }
    }
    fwht<64>(v);
    uint32_t words[FP8OUT ? 16 : 8];
    uint32_t sbytes;
    mx_encode64<64, FP8OUT>(v, words, sbytes);
    const int row = m0 + wm * 128 + lrow;
    const int col = n0 + wn * 128 + 64 * half;
    if (row < p.M && col < p.N) {
      constexpr int BYTES = FP8OUT ? 64 : 32;
      uint4* q = reinterpret_cast<uint4*>(p.q_out + (int64_t)row * (FP8OUT ? p.N : p.N / 2) + (FP8OUT ? col : col / 2));
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i) q[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
      *reinterpret_cast<uint16_t*>(p.s_out + (int64_t)row * (p.N / 32) + col / 32) = (uint16_t)sbytes;
    }
  }
}

// STAGED: the bf16 epilogue through LDS (the host checks staged_store_ok);
// otherwise per-element stores.  QOUT 1 / 2: the quantizing epilogue with
// MXFP4 / MXFP8 codes (the GELU table sits after the ring).  One epilogue
// per instantiation keeps the accumulators in AGPRs until they are read.
template <bool A8, bool QUADS, bool SPLIT, bool STAGED, int QOUT = 0>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm_mx_kernel(GemmParams p) {
  using P = MxPipe<A8, QUADS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = p.K;

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

  const uint8_t* aq = static_cast<const uint8_t*>(p.a_q);
  const uint8_t* as = static_cast<const uint8_t*>(p.a_s);

  // ---- per-lane byte offsets of the loads at k0 = 0 (32-bit: every operand
  // matrix is below 4 GB, checked on the host); rows past M / N repeat the
  // last row and are never stored
  uint32_t offA[P::NA], offW[P::NW];
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
  for (int u = 0; u < P::NW; ++u) {
    const int r = (wv * P::NW + u) * 16 + (lane >> 2);
    const int q = (lane & 3) ^ ((r >> 1) & 3);
    offW[u] = (uint32_t)min(n0 + r, p.N - 1) * (uint32_t)(K / 2) + 16u * q;
  }
  const uint32_t offAS = (uint32_t)min(m0 + wv * 64 + lane, p.M - 1) * (uint32_t)(K / 32);
  const uint32_t offWS = (uint32_t)min(n0 + wv * 64 + lane, p.N - 1) * (uint32_t)(K / 32);

  const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t*)smem;
  const uint32_t wvu = __builtin_amdgcn_readfirstlane(wv);
  auto slot = [&](int kt) { return (kt - kb) % P::NS; };
  auto issue_stage = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)slot(kt) * P::STAGE;
    const int k0 = kt * BK;
    const uint8_t* abase = aq + (A8 ? k0 : k0 / 2);
    const uint8_t* wbase = p.w_q + k0 / 2;
#pragma unroll
    for (int u = 0; u < P::NA; ++u) dma16(abase, offA[u], st + (wvu * P::NA + u) * 1024);
#pragma unroll
    for (int u = 0; u < P::NW; ++u) dma16(wbase, offW[u], st + P::A_CODES + (wvu * P::NW + u) * 1024);
    if constexpr (QUADS) {
      // the 16 scale bytes of stages 4g .. 4g+3 per row, into buffer g % 2
      // (a slice that starts inside a quad loads that quad first)
      if ((kt & 3) == 0 || kt == kb) {
        const uint32_t sq = lds0 + P::SQ + (uint32_t)((kt >> 2) & 1) * 8192u + wvu * 1024u;
        dma16(as + (kt >> 2) * 16, offAS, sq);
        dma16(p.w_s + (kt >> 2) * 16, offWS, sq + 4096u);
      }
    } else {
      dma4(as + k0 / 32, offAS, st + P::A_CODES + P::W_CODES + wvu * 256);
      dma4(p.w_s + k0 / 32, offWS, st + P::A_CODES + P::W_CODES + P::A_SC + wvu * 256);
    }
  };

  const int r32 = lane & 31, h = lane >> 5;
  // fragments of step s (k = 64 s .. +63 of the stage)
  auto read_frag = [&](int kt, int s, MxFrag<A8>& F) {
    const uint8_t* st = smem + slot(kt) * P::STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + r32;
      if constexpr (A8) {
        const int4v lo = *reinterpret_cast<const int4v*>(st + i8_quad_off(row, 4 * s + h));
        const int4v hi = *reinterpret_cast<const int4v*>(st + i8_quad_off(row, 4 * s + 2 + h));
        F.a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        F.a[i] = *reinterpret_cast<const int4v*>(st + fp4_quad_off(row, 2 * s + h));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + 32 * j + r32;
      F.w[j] = *reinterpret_cast<const int4v*>(st + P::A_CODES + fp4_quad_off(row, 2 * s + h));
    }
  };
  // the scale dwords of a stage (4 blocks of each fragment row); a lane uses
  // them shifted right by 8 (lane / 32) bits, so that byte 0 / 2 is its
  // block of step 0 / 1
  // (with QUADS: the 16 bytes of the stage's quad; pick_scale takes the
  // stage's dword)
  using ScaleReg = std::conditional_t<QUADS, int4v, uint32_t>;
  auto read_scales = [&](int kt, ScaleReg (&sa)[4], ScaleReg (&sw)[4]) {
    if constexpr (QUADS) {
      const uint8_t* sq = smem + P::SQ + ((kt >> 2) & 1) * 8192;
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = *reinterpret_cast<const int4v*>(sq + 16 * (wm * 128 + 32 * i + r32));
#pragma unroll
      for (int j = 0; j < 4; ++j) sw[j] = *reinterpret_cast<const int4v*>(sq + 4096 + 16 * (wn * 128 + 32 * j + r32));
    } else {
      const uint8_t* st = smem + slot(kt) * P::STAGE + P::A_CODES + P::W_CODES;
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(st + 4 * (wm * 128 + 32 * i + r32));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sw[j] = *reinterpret_cast<const uint32_t*>(st + P::A_SC + 4 * (wn * 128 + 32 * j + r32));
    }
  };
  auto pick_scale = [&](const ScaleReg& r, int kt) -> uint32_t {
    if constexpr (QUADS) {
      const int j = kt & 3;
      return (uint32_t)(j == 0 ? r[0] : j == 1 ? r[1] : j == 2 ? r[2] : r[3]);
    } else {
      return r;
    }
  };
  const uint32_t hsh = 8 * h;

  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // D = W_frag x A_frag^T: each accumulator tile is a 32 x 32 block of Y^T,
  // so a lane holds one token row and, per register group of 4, four
  // consecutive output features (vector stores in the epilogue)
  auto mfma16 = [&](const MxFrag<A8>& F, const uint32_t (&sa)[4], const uint32_t (&sw)[4], auto opsel) {
    constexpr int OP = decltype(opsel)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            mx_operand(F.w[j]), mx_operand(F.a[i]), acc[i][j], kMfmaFp4, A8 ? kMfmaFp8 : kMfmaFp4, OP,
            (int)sw[j], OP, (int)sa[i]);
  };

  // interleave each matrix instruction of a step with one LDS read (the next
  // step's fragments or scales) and a shift; each step is its own
  // scheduling region
  auto interleave = [&]() {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: every ring slot loading, wait for the first stage
  const int pre = min(P::NS, ke - kb);
  for (int s = 0; s < pre; ++s) issue_stage(kb + s);
  if constexpr (QOUT != 0) {
    // copied under the first loads; the loop's barriers order it before use
    if (p.qflags & 4u) {
      for (int i = threadIdx.x; i < kGeluTabBytes / 16; i += GT)
        reinterpret_cast<uint4*>(smem + P::GTAB)[i] = reinterpret_cast<const uint4*>(p.gtab)[i];
    }
  }
  wait_stages<P::LPS>(pre - 1);
  wait_lgkm_barrier();

  MxFrag<A8> F0, F1;
  ScaleReg ra[4], rw[4];                 // scale dwords (or quads) as read
  uint32_t sa[4], sw[4];                 // the stage's dwords, shifted
  read_scales(kb, ra, rw);
  read_frag(kb, 0, F0);

  for (int kt = kb; kt < ke; ++kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { sa[i] = pick_scale(ra[i], kt) >> hsh; sw[i] = pick_scale(rw[i], kt) >> hsh; }
    // step 0 | read step 1
    read_frag(kt, 1, F1);
    mfma16(F0, sa, sw, std::integral_constant<int, 0>{});
    interleave();
    // every read of stage kt issued: wait for them and for this wave's loads
    // of stage kt+1; after the barrier stage kt+1 is complete in LDS and
    // stage kt's slot is free for stage kt+NS
    wait_stages<P::LPS>(min(P::NS - 2, ke - kt - 2));
    wait_lgkm_barrier();
    if (kt + P::NS < ke) issue_stage(kt + P::NS);
    // step 1 | read stage kt+1's scales and step 0 (a stale slot past the
    // last stage: read, never used)
    mfma16(F1, sa, sw, std::integral_constant<int, 2>{});
    read_scales(kt + 1, ra, rw);
    read_frag(kt + 1, 0, F0);
    interleave();
  }

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

  if constexpr (QOUT != 0) {
    quant_store_tile<QOUT == 2>(p, acc, smem, reinterpret_cast<const uint16_t*>(smem + P::GTAB), m0, n0);
    return;
  }
  // bf16 output in whole 16-byte chunks: through LDS (the ring is free)
  if constexpr (STAGED) {
    stage_store_tile<2, (P::LDS >= 4 * 32768) ? 1 : 2>(p, acc, smem, m0, n0);
    return;
  }
  // epilogue: tile (i, j), lane, register e -> token row m0 + wm*128 + 32 i
  // + lane%32, feature column n0 + wn*128 + 32 j + 8 (e/4) + 4 (lane/32) + e%4
  const bool vec = out_vec_ok(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + 32 * i + r32;
    if (row >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        emit4(p, vec, row, n0 + wn * 128 + 32 * j + 8 * g + 4 * h, 1.0f, acc[i][j][4 * g],
              acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
  }
}

template <bool A8, bool QUADS, bool SPLIT, bool STAGED, int QOUT = 0>
static size_t mx_lds_bytes() {
  return QOUT ? (size_t)MxPipe<A8, QUADS>::GTAB + kGeluTabBytes : (size_t)MxPipe<A8, QUADS>::LDS;
}

template <bool A8, bool QUADS, bool SPLIT, bool STAGED, int QOUT = 0>
static hipError_t set_mx_lds_attr() {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qgemm_mx_kernel<A8, QUADS, SPLIT, STAGED, QOUT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)mx_lds_bytes<A8, QUADS, SPLIT, STAGED, QOUT>());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

template <bool A8, bool QUADS>
static hipError_t launch_mx(GemmParams p, hipStream_t st) {
  int dp_grid = 0, sk_grid = 0;
  plan_pipe(p, cu_count(), dp_grid, sk_grid);
  const size_t lds = (size_t)MxPipe<A8, QUADS>::LDS;
  // the same test as the device-side staged_store_ok
  const bool staged = !p.out_f32 && (p.N % 8) == 0 && (p.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15u) == 0 &&
                      (!p.bias || (reinterpret_cast<uintptr_t>(p.bias) & 15u) == 0);
  hipError_t e = staged ? set_mx_lds_attr<A8, QUADS, false, true>() : set_mx_lds_attr<A8, QUADS, false, false>();
  if (e == hipSuccess) e = set_mx_lds_attr<A8, QUADS, true, false>();
  if (e != hipSuccess) return e;
  if (dp_grid > 0) {
    if (staged)
      hipLaunchKernelGGL((qgemm_mx_kernel<A8, QUADS, false, true>), dim3(dp_grid), dim3(GT), lds, st, p);
    else
      hipLaunchKernelGGL((qgemm_mx_kernel<A8, QUADS, false, false>), dim3(dp_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sk_grid > 0) {
    hipLaunchKernelGGL((qgemm_mx_kernel<A8, QUADS, true, false>), dim3(sk_grid), dim3(GT), lds, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((qgemm_reduce_kernel<2>), dim3(p.sk_tiles * 64), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

// Quantizing variant: every tile in the data-parallel kernel (no K split).
template <bool A8, bool QUADS, int QOUT>
static hipError_t launch_mx_quant(GemmParams p, hipStream_t st) {
  int dp_grid = 0, sk_grid = 0;
  plan_pipe(p, cu_count(), dp_grid, sk_grid);
  p.sk_tiles = 0;
  p.slices = 0;
  p.slice_nk = 0;
  dp_grid = p.tiles_m * p.tiles_n;
  hipError_t e = set_mx_lds_attr<A8, QUADS, false, false, QOUT>();
  if (e != hipSuccess) return e;
  const size_t lds = mx_lds_bytes<A8, QUADS, false, false, QOUT>();
  hipLaunchKernelGGL((qgemm_mx_kernel<A8, QUADS, false, false, QOUT>), dim3(dp_grid), dim3(GT), lds, st, p);
  return hipGetLastError();
}

// Scale quads need 16-byte aligned 16-byte runs in every scale row.
static bool mx_quads(int64_t K) { return K % 512 == 0; }

hipError_t launch_qgemm_mx_quant(bool a_fp8, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                                 const uint8_t* w_s, const float* bias, bool out_fp8, bool gelu, uint8_t* q_out,
                                 uint8_t* s_out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_ts = nullptr;
  p.w_q = w_q; p.w_s = w_s; p.w_ts = nullptr;
  p.bias = bias; p.y = nullptr; p.ldy = 0;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.q_out = q_out; p.s_out = s_out; p.qflags = gelu ? 4u : 0u;
  if (gelu) {
    const hipError_t e = gelu_table(st, &p.gtab);
    if (e != hipSuccess) return e;
  }
  if (mx_quads(K)) {
    if (a_fp8) return out_fp8 ? launch_mx_quant<true, true, 2>(p, st) : launch_mx_quant<true, true, 1>(p, st);
    return out_fp8 ? launch_mx_quant<false, true, 2>(p, st) : launch_mx_quant<false, true, 1>(p, st);
  }
  if (a_fp8) return out_fp8 ? launch_mx_quant<true, false, 2>(p, st) : launch_mx_quant<true, false, 1>(p, st);
  return out_fp8 ? launch_mx_quant<false, false, 2>(p, st) : launch_mx_quant<false, false, 1>(p, st);
}

hipError_t launch_qgemm_mx(bool a_fp8, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                           const uint8_t* w_s, const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                           int64_t N, int64_t K, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_ts = nullptr;
  p.w_q = w_q; p.w_s = w_s; p.w_ts = nullptr;
  p.bias = bias; p.y = y; p.ldy = ldy;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.out_f32 = out_dtype == 1;
  p.part = static_cast<float*>(ws);
  if (mx_quads(K)) return a_fp8 ? launch_mx<true, true>(p, st) : launch_mx<false, true>(p, st);
  return a_fp8 ? launch_mx<true, false>(p, st) : launch_mx<false, false>(p, st);
}

}  // namespace vdtq
