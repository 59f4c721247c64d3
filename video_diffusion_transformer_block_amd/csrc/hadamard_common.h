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
// function of 16 bits, and its sign is the input's (GELU(x) = x times a
// positive factor; negative results that round to zero stay -0).  Over all
// finite bf16 x (checked exhaustively): |RNE_bf16(gelu_fp32(x))| =
// |RNE_bf16(x / 2)| when |x| < 2^-9 (magnitude bits below 0x3b00; for
// magnitude bits >= 0x100 that is one less in the exponent field), |x| when
// x >= 2.75 (0x4030), and 0 when x <= -10.0625 (0xc121).
//
// The lookup works on a 32-bit word of two bf16 values with packed 16-bit
// arithmetic.  Each value's magnitude bits m select a table entry holding a
// subtrahend s, and the result is sign | max(m - s, 0):
//   index = min(m, 0x100) + clamp(m - (0x3b00 - 1), 0, 1570) + sign * 1827
// selects, within the sign's 1827 entries:
//   m itself for m < 0x100 (subnormal and the smallest normal inputs,
//     whose halving rounds);
//   0x100 for the rest below 0x3b00 (s = 0x80: one less in the exponent
//     field; 0 stays 0 by the clamp at zero);
//   0x101 + (m - 0x3b00) for 0x3b00 <= m < 0x4121 (s = m - |GELU|; 0 for
//     the positive inputs from 0x4030 up, where GELU(x) = x);
//   the last entry for m >= 0x4121 (0 for positive inputs, 0x7fff for
//     negative ones, whose GELU is -0).
constexpr int kGeluLo = 0x3B00, kGeluLim = 0x4121 - 0x3B00 + 1;   // clamp bound 1570
constexpr int kGeluRegion = 0x101 + kGeluLim;                       // entries per sign
constexpr int kGeluTabN = 2 * kGeluRegion;
constexpr int kGeluTabBytes = ((2 * kGeluTabN + 15) / 16) * 16;

// Table entry i (0 <= i < kGeluTabN): the subtrahend of the inputs that
// map to it, from one representative input.
__device__ __forceinline__ uint16_t gelu_table_entry(int i) {
  const uint32_t sign = i >= kGeluRegion ? 0x8000u : 0u;
  const int e = i - (sign ? kGeluRegion : 0);
  if (sign && e == kGeluRegion - 1) return 0x7FFFu;                 // large negative: -0
  const uint32_t m = e <= 0x100 ? (uint32_t)e : (uint32_t)(kGeluLo + (e - 0x101));
  const uint32_t g = f32_to_bf16_bits(gelu_fp32(__uint_as_float((sign | m) << 16)));
  return (uint16_t)(m - (g & 0x7FFFu));
}

typedef short short2v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

// RNE_bf16(gelu_fp32(x)) for both bf16 values of w (low half first), from
// the table above (finite inputs).
__device__ __forceinline__ uint32_t gelu_word(uint32_t w, const uint16_t* tab) {
  const uint32_t mag = w & 0x7FFF7FFFu;
  const ushort2v m = __builtin_bit_cast(ushort2v, mag);
  short2v d = __builtin_bit_cast(short2v, mag) - (short2v)(short)(kGeluLo - 1);   // |d| < 2^15
  d = __builtin_elementwise_max(__builtin_elementwise_min(d, (short2v)(short)kGeluLim), (short2v)(short)0);
  const ushort2v sign = __builtin_bit_cast(ushort2v, w) >> (ushort2v)(unsigned short)15;
  const ushort2v idx = __builtin_elementwise_min(m, (ushort2v)(unsigned short)0x100) +
                       __builtin_bit_cast(ushort2v, d) + sign * (ushort2v)(unsigned short)kGeluRegion;
  const uint32_t iw = __builtin_bit_cast(uint32_t, idx);
  const ushort2v s = {tab[iw & 0xFFFFu], tab[iw >> 16]};
  const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(m, s));
  return r | (w & 0x80008000u);
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
