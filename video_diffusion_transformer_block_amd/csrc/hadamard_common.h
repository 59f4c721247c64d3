// Per-thread pieces of the activation transform shared by the standalone
// quantize pass (hadamard_quantize.hip) and the quantizing epilogue of the
// MX GEMM (qgemm_mx.hip): the fp32 GELU of the DiT feed-forward, the block
// Hadamard butterflies on a thread's 64 register values, and the MX
// (E8M0-scaled E2M1 / E4M3) encoding of two 32-element blocks.
//
// The operations: gist.science "6Bit-Diffusion: Inference-Time
// Mixed-Precision Quantization for Video Diffusion Models" §2.A (block
// Hadamard before quantization) and §4 (quantization fused into the
// producing kernel); OCP Microscaling v1.0 §6.3 (the MX conversion).  All
// arithmetic is fp32 round-to-nearest-even with contraction disabled.
#pragma once

#include "device_common.h"

namespace vdtq {

// ---------------------------------------------------------------- GELU
// GELU, tanh form, as y * sigmoid(2u) = y / (1 + e^(-2u)) with
// u = sqrt(2/pi) (y + 0.044715 y^3), every step one fp32 operation:
//   u = C0 * (y + C1 * ((y * y) * y)),  z = clamp(-2 u, -80, 90),
//   GELU = y / (1 + exp(z))           (correctly rounded division)
// exp: k = rint(z / ln 2) (z times RN(1/ln 2)), r = (z - k L_hi) - k L_lo
// with L_hi = ln 2 cut to 12 significant bits (k L_hi exact), the degree-7
// Taylor polynomial of e^r in Horner form with coefficients RN(1/n!), and
// two exact scalings by 2^floor(k/2) and 2^(k - floor(k/2)): z = 90
// overflows to +inf (GELU -> -0), z = -80 stays normal (GELU -> y).
constexpr float kGeluC0 = 0x1.988454p-1f;     // RN(sqrt(2/pi))
constexpr float kGeluC1 = 0x1.6e4e26p-5f;     // RN(0.044715)
constexpr float kLog2e = 0x1.715476p+0f;      // RN(1/ln 2)
constexpr float kLn2Hi = 0x1.62ep-1f;
constexpr float kLn2Lo = 0x1.0bfbe8p-15f;     // RN(ln 2 - kLn2Hi)

__device__ __forceinline__ float exp_fp32(float z) {
  const float k = __builtin_rintf(z * kLog2e);
  const float r = (z - k * kLn2Hi) - k * kLn2Lo;
  float q = 0x1.a01a02p-13f;                   // 1/7!
  q = q * r + 0x1.6c16c2p-10f;                 // 1/6!
  q = q * r + 0x1.111112p-7f;                  // 1/5!
  q = q * r + 0x1.555556p-5f;                  // 1/4!
  q = q * r + 0x1.555556p-3f;                  // 1/3!
  q = q * r + 0.5f;
  q = q * r + 1.0f;
  q = q * r + 1.0f;
  const int ki = (int)k;
  const int k1 = ki >> 1;                      // floor(k / 2)
  return ldexpf(ldexpf(q, k1), ki - k1);
}

__device__ __forceinline__ float gelu_fp32(float y) {
  const float y3 = (y * y) * y;
  const float u = kGeluC0 * (y + kGeluC1 * y3);
  float z = -2.0f * u;
  z = z < -80.0f ? -80.0f : (z > 90.0f ? 90.0f : z);
  return y / (1.0f + exp_fp32(z));
}

// The kernels apply GELU to bf16 inputs and keep a bf16 result, so it is a
// function of 16 bits; they evaluate gelu_fp32 once per workgroup for the
// inputs where it is not trivial and look the rest up.  Over all finite
// bf16 x (checked exhaustively): RNE_bf16(gelu_fp32(x)) equals
// RNE_bf16(x / 2) when |x| < 2^-9 (bits & 0x7fff below 0x3b00), x itself
// when x >= 2.75 (0x4030), and -0 when x <= -10.0625 (0xc121).  The table
// holds the positive inputs 0x3b00 .. 0x402f, then the negative ones
// 0xbb00 .. 0xc120.  Inputs are finite.
constexpr uint32_t kGeluLo = 0x3B00u, kGeluPosEnd = 0x4030u, kGeluNegEnd = 0x4121u;
constexpr int kGeluPosN = (int)(kGeluPosEnd - kGeluLo);
constexpr int kGeluTabN = kGeluPosN + (int)(kGeluNegEnd - kGeluLo);
constexpr int kGeluTabBytes = ((2 * kGeluTabN + 15) / 16) * 16;

// Table entry i (0 <= i < kGeluTabN).
__device__ __forceinline__ uint16_t gelu_table_entry(int i) {
  const uint32_t b = i < kGeluPosN ? kGeluLo + i : (0x8000u | (kGeluLo + (i - kGeluPosN)));
  return (uint16_t)f32_to_bf16_bits(gelu_fp32(__uint_as_float(b << 16)));
}

// Fills the table; every thread of the workgroup takes part (a barrier
// must follow before the first lookup).
__device__ __forceinline__ void gelu_table_build(uint16_t* tab) {
  for (int i = threadIdx.x; i < kGeluTabN; i += blockDim.x) tab[i] = gelu_table_entry(i);
}

// RNE_bf16(gelu_fp32(x)) for the bf16 bits b of a finite x.  Below the
// table, x / 2 is exact for exponent fields >= 2 (one less in the exponent
// field); smaller inputs round (rare: a divergent branch).
__device__ __forceinline__ uint32_t gelu_bf16_bits(uint32_t b, const uint16_t* tab) {
  const uint32_t mag = b & 0x7FFFu;
  const bool neg = b > 0x7FFFu;
  const uint32_t idx = mag - kGeluLo;                       // wraps below the table
  const bool in_tab = idx < (neg ? kGeluNegEnd - kGeluLo : kGeluPosEnd - kGeluLo);
  const uint32_t t = tab[in_tab ? idx + (neg ? (uint32_t)kGeluPosN : 0u) : 0u];
  uint32_t r = neg ? 0x8000u : b;                           // above the table
  if (mag < kGeluLo) {
    r = b - 0x80u;
    if (mag < 0x100u) r = f32_to_bf16_bits(__uint_as_float(b << 16) * 0.5f);
  }
  return in_tab ? t : r;
}

// ---------------------------------------------------------------- Hadamard
// Butterflies in the fixed order h = 1, 2, ..., b/2 (fp32, RNE).
template <int B>
__device__ __forceinline__ void fwht(float (&v)[64]) {
  constexpr int HIN = B < 64 ? B : 64;
#pragma unroll
  for (int h = 1; h < HIN; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  // stages across chunks: h = 64 pairs lanes t, t^1; h = 128 pairs t, t^2.
  if (B >= 128) {
    const bool upper = threadIdx.x & 1;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      float o = __shfl_xor(v[i], 1, 64);
      v[i] = upper ? (o - v[i]) : (v[i] + o);
    }
  }
  if (B >= 256) {
    const bool upper = threadIdx.x & 2;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      float o = __shfl_xor(v[i], 2, 64);
      v[i] = upper ? (o - v[i]) : (v[i] + o);
    }
  }
}

// Normalisation.  Powers of four keep v unscaled (y = v * 2^-k exactly, the
// factor is folded downstream); b = 32 / 128 multiply by RN(1/sqrt(b)) here.
template <int B> struct HadScale;
template <> struct HadScale<16>  { static constexpr bool pow4 = true;  static constexpr float f = 0.25f;    static constexpr float inv = 4.0f; };
template <> struct HadScale<64>  { static constexpr bool pow4 = true;  static constexpr float f = 0.125f;   static constexpr float inv = 8.0f; };
template <> struct HadScale<256> { static constexpr bool pow4 = true;  static constexpr float f = 0.0625f;  static constexpr float inv = 16.0f; };
// RN_fp32(sqrt 2) = 0x1.6a09e6p+0; 1/sqrt(32) = sqrt(2)/8, 1/sqrt(128) = sqrt(2)/16
template <> struct HadScale<32>  { static constexpr bool pow4 = false; static constexpr float f = 0x1.6a09e6p-3f; static constexpr float inv = 1.0f; };
template <> struct HadScale<128> { static constexpr bool pow4 = false; static constexpr float f = 0x1.6a09e6p-4f; static constexpr float inv = 1.0f; };

template <int B>
__device__ __forceinline__ void normalise(float (&v)[64]) {
  if (!HadScale<B>::pow4) {
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = v[i] * HadScale<B>::f;
  }
}
// factor from the register values to y (1 when already applied)
template <int B>
__device__ __forceinline__ constexpr float yfac() { return HadScale<B>::pow4 ? HadScale<B>::f : 1.0f; }

// ---------------------------------------------------------------- MX
// E8M0 exponent e of a 32-element block from the maximum |v| of its register
// values (y = v * 2^-KSH): e = floor(log2 max|y|) - EMAX clamped to
// [-127, 127]; zero (and fp32-subnormal maxima, whose e clamps anyway) give
// -127.
template <int EMAX, int KSH>
__device__ __forceinline__ int mx_exponent(float amax_v) {
  const int ex = (int)((__float_as_uint(amax_v) >> 23) & 0xFFu);
  if (ex == 0) return -127;
  return min(max(ex - 127 - KSH - EMAX, -127), 127);
}

// 2^n as fp32 for n in [-126, 127] (exact)
__device__ __forceinline__ float exp2i(int n) { return __uint_as_float((uint32_t)(n + 127) << 23); }

// log2 of the power-of-two factor from register values to y (0 when the
// normalisation is already applied)
template <int B> struct HadShift { static constexpr int k = 0; };
template <> struct HadShift<16>  { static constexpr int k = 2; };
template <> struct HadShift<64>  { static constexpr int k = 3; };
template <> struct HadShift<256> { static constexpr int k = 4; };

// MX encoding of a thread's 64 values (two 32-element blocks, register
// values v = y * 2^KSH): E2M1 codes (4 words per block, low nibble first) or
// E4M3 codes (8 words per block), and the two E8M0 scale bytes in the low
// 16 bits of sbytes.
template <int B, bool FP8>
__device__ __forceinline__ void mx_encode64(const float (&v)[64], uint32_t (&words)[FP8 ? 16 : 8], uint32_t& sbytes) {
  constexpr int KSH = HadShift<B>::k;
  constexpr int EMAX = FP8 ? 8 : 2;
  sbytes = 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float* vb = &v[32 * blk];
    float av = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) av = fmaxf(av, fabsf(vb[e]));
    const int e = mx_exponent<EMAX, KSH>(av);
    sbytes |= (uint32_t)(e + 127) << (8 * blk);
    // t = v * 2^-(e + KSH) as two exact power-of-two factors, each a normal
    // fp32 (|n1|, |n2| <= 65); an intermediate that underflows belongs to an
    // element far below the smallest nonzero code
    const int n = e + KSH;
    const int n1 = n / 2, n2 = n - n1;
    const float m1 = exp2i(-n1), m2 = exp2i(-n2);
    if constexpr (FP8) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = __builtin_amdgcn_fmed3f((vb[4 * w + i] * m1) * m2, -448.0f, 448.0f);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], x, true);
        words[8 * blk + w] = (uint32_t)x;
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t x = 0u;
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, (vb[8 * w + 0] * m1) * m2, (vb[8 * w + 1] * m1) * m2, 1.0f, 0);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, (vb[8 * w + 2] * m1) * m2, (vb[8 * w + 3] * m1) * m2, 1.0f, 1);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, (vb[8 * w + 4] * m1) * m2, (vb[8 * w + 5] * m1) * m2, 1.0f, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, (vb[8 * w + 6] * m1) * m2, (vb[8 * w + 7] * m1) * m2, 1.0f, 3);
        words[4 * blk + w] = x;
      }
    }
  }
}

}  // namespace vdtq
