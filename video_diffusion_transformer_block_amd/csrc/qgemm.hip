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
// Tiling: 256 threads = 4 wavefronts in a 2 x 2 arrangement, a 128 x 128
// output tile per workgroup, 64 x 64 per wavefront (2 x 2 MFMA 32x32 tiles),
// K consumed 64 at a time.  Each thread loads 32 packed elements of one row of
// A and of W, decodes them (hardware fp4 -> f16 conversion, then one packed
// f16 multiply by the group scale; int8 -> f16 by the 0x6400 bias trick) and
// writes them to LDS, from where the wavefronts read MFMA fragments with
// 16-byte LDS reads.
#include "device_common.h"
#include "launch.h"

namespace vdtq {

constexpr int GT = 256;          // threads
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK + 8;     // padded row (halves): 144 B, conflict-free 16-B reads

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
};

// e4m3 byte -> fp16 pair (exact: e4m3 values lie in fp16's range)
__device__ __forceinline__ half2v scale_pair(uint32_t s8) {
  _Float16 h = (_Float16)e4m3_decode_pos(s8);
  return half2v{h, h};
}

// 8 e2m1 codes (one dword) * fp16 scale -> 8 halves (exact products)
__device__ __forceinline__ void dec_fp4x8(uint32_t w, half2v s, half2v* out) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
}

// 4 int8 (one dword) -> 4 halves: fp16 0x6400 | (b ^ 0x80) is 1024 + b + 128
__device__ __forceinline__ void dec_i8x4(uint32_t w, half2v* out) {
  const uint32_t x = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
  const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  out[0] = __builtin_bit_cast(half2v, lo) - bias;
  out[1] = __builtin_bit_cast(half2v, hi) - bias;
}

// Loads and decodes 32 consecutive NVFP4 elements (k0 .. k0+31) of one row.
__device__ __forceinline__ void load_dec_fp4_row(const uint8_t* q, const uint8_t* s, int64_t row,
                                                 int K, int k0, half2v (&h)[16]) {
  const uint8_t* qr = q + row * (K / 2) + k0 / 2;
  const uint8_t* sr = s + row * (K / 16) + k0 / 16;
  uint4 w = make_uint4(0u, 0u, 0u, 0u);
  uint32_t s0 = 0u, s1 = 0u;
  if (k0 + 32 <= K) {
    if ((K & 31) == 0) {
      w = *reinterpret_cast<const uint4*>(qr);
    } else {   // rows of K/2 bytes are only 8-byte aligned
      uint2 a = reinterpret_cast<const uint2*>(qr)[0], b = reinterpret_cast<const uint2*>(qr)[1];
      w = make_uint4(a.x, a.y, b.x, b.y);
    }
    s0 = sr[0];
    s1 = sr[1];
  } else if (k0 + 16 <= K) {
    uint2 w2 = *reinterpret_cast<const uint2*>(qr);
    w.x = w2.x;
    w.y = w2.y;
    s0 = sr[0];
  }
  const half2v sc0 = scale_pair(s0), sc1 = scale_pair(s1);
  dec_fp4x8(w.x, sc0, &h[0]);
  dec_fp4x8(w.y, sc0, &h[4]);
  dec_fp4x8(w.z, sc1, &h[8]);
  dec_fp4x8(w.w, sc1, &h[12]);
}

__device__ __forceinline__ void load_dec_i8_row(const int8_t* q, int64_t row, int K, int k0,
                                                half2v (&h)[16]) {
  const int8_t* qr = q + row * K + k0;
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
  if (k0 + 16 <= K) a = *reinterpret_cast<const uint4*>(qr);
  if (k0 + 32 <= K) b = *reinterpret_cast<const uint4*>(qr + 16);
  dec_i8x4(a.x, &h[0]); dec_i8x4(a.y, &h[2]); dec_i8x4(a.z, &h[4]); dec_i8x4(a.w, &h[6]);
  dec_i8x4(b.x, &h[8]); dec_i8x4(b.y, &h[10]); dec_i8x4(b.z, &h[12]); dec_i8x4(b.w, &h[14]);
}

template <int AFMT>
__global__ __launch_bounds__(GT) void qgemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) _Float16 Ws[BN * LDSK];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  // loader role: row r of the tile, k half kh
  const int r = t >> 1, kh = t & 1;
  const int64_t arow = min(m0 + r, p.M - 1);   // clamped; rows >= M never stored
  const int64_t wrow = min(n0 + r, p.N - 1);

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  for (int k0 = 0; k0 < p.K; k0 += BK) {
    half2v ha[16], hw[16];
    const int kk = k0 + 32 * kh;
    if (AFMT == 0)
      load_dec_fp4_row(static_cast<const uint8_t*>(p.a_q), static_cast<const uint8_t*>(p.a_s), arow,
                       p.K, kk, ha);
    else
      load_dec_i8_row(static_cast<const int8_t*>(p.a_q), arow, p.K, kk, ha);
    load_dec_fp4_row(p.w_q, p.w_s, wrow, p.K, kk, hw);

    __syncthreads();   // previous iteration's fragment reads are done
    uint4* adst = reinterpret_cast<uint4*>(&As[r * LDSK + 32 * kh]);
    uint4* wdst = reinterpret_cast<uint4*>(&Ws[r * LDSK + 32 * kh]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      adst[i] = __builtin_bit_cast(uint4, half8{ha[4 * i][0], ha[4 * i][1], ha[4 * i + 1][0], ha[4 * i + 1][1],
                                                ha[4 * i + 2][0], ha[4 * i + 2][1], ha[4 * i + 3][0], ha[4 * i + 3][1]});
      wdst[i] = __builtin_bit_cast(uint4, half8{hw[4 * i][0], hw[4 * i][1], hw[4 * i + 1][0], hw[4 * i + 1][1],
                                                hw[4 * i + 2][0], hw[4 * i + 2][1], hw[4 * i + 3][0], hw[4 * i + 3][1]});
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const half8*>(
            &As[(wm * 64 + 32 * i + (lane & 31)) * LDSK + 16 * ks + 8 * (lane >> 5)]);
        bf[i] = *reinterpret_cast<const half8*>(
            &Ws[(wn * 64 + 32 * i + (lane & 31)) * LDSK + 16 * ks + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: C[row][col] of MFMA tile (i, j): lane, register e ->
  // row 8*(e/4) + 4*(lane/32) + e%4, col lane%32
  const float gsw = p.w_ts[1];
  const float alpha_t = (AFMT == 0) ? p.a_ts[1] * gsw : 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (row >= p.M) continue;
      const float alpha = (AFMT == 0) ? alpha_t : static_cast<const float*>(p.a_s)[row] * gsw;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + 32 * j + (lane & 31);
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

hipError_t launch_qgemm(int afmt, const void* a_q, const void* a_s, const float* a_ts,
                        const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                        const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                        int64_t N, int64_t K, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{a_q, a_s, a_ts, w_q, w_s, w_ts, bias, y, ldy, (int32_t)M, (int32_t)N, (int32_t)K,
               out_dtype == 1};
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (afmt == 0)
    hipLaunchKernelGGL(qgemm_kernel<0>, grid, dim3(GT), 0, st, p);
  else
    hipLaunchKernelGGL(qgemm_kernel<1>, grid, dim3(GT), 0, st, p);
  return hipGetLastError();
}

}  // namespace vdtq
