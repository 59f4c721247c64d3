// Device helpers for the gfx950 kernels: bf16 / E4M3 bit conversions, the
// NVFP4 tensor-scale recipe, and deterministic wavefront reductions.
//
// Every helper is written from the format definitions (IEEE binary32,
// OCP 8-bit FP E4M3 "fn", OCP MX FP4 E2M1); none is shared with the CPU
// oracle.  All arithmetic relies on fp32 round-to-nearest-even with
// contraction disabled (-ffp-contract=off) and correctly rounded division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdtq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Threshold below which a tensor (NVFP4) or a row (INT8) quantizes to zero:
// scales derived from smaller maxima would leave the fp32 normal range.
constexpr float kZeroLimit = 0x1p-100f;

// Raw (unstrided, unswizzled) buffer resources over [p, p + bytes): the
// hardware's range check makes loads past the end read zeros and drops
// stores past it, so bounded accesses need no branch.  Word 3 selects the
// 32-bit data format, which untyped accesses need to move anything.
constexpr int kRawBufferWord3 = 0x00020000;
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRawBufferWord3);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const uint4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float buffer_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 w) {
  const uint4v v = {w.x, w.y, w.z, w.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// The double whose bits are (hi:lo).
__device__ __forceinline__ double u2d(uint32_t lo, uint32_t hi) {
  return __hiloint2double((int)hi, (int)lo);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-negative finite fp32 -> OCP E4M3 byte, nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0x1p-6f) {
    // subnormal range: integer number of 2^-9 units, ties to even via the
    // 2^23 magic constant (t < 8, so t + 2^23 rounds at unit 1)
    float t = s * 512.0f;
    float r = (t + 8388608.0f) - 8388608.0f;
    return (uint32_t)r;  // 8 encodes 2^-6, the smallest normal
  }
  uint32_t u = __float_as_uint(s);
  u += 0x7FFFFu + ((u >> 20) & 1u);            // round mantissa to 3 bits
  uint32_t code = (u >> 20) - (120u << 3);     // rebias exponent 127 -> 7
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 byte (sign ignored, finite) -> fp32, exact.
__device__ __forceinline__ float e4m3_decode_pos(uint32_t b) {
  uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// NVFP4 tensor scale: gs = RN(amax / 2688) when amax is usable, else 1.
__device__ __forceinline__ bool nvfp4_amax_ok(float amax) {
  return (amax == amax) && amax >= kZeroLimit && amax <= 3.0e38f;
}
__device__ __forceinline__ float nvfp4_gs(float amax) {
  return nvfp4_amax_ok(amax) ? amax / 2688.0f : 1.0f;
}

// ---------------------------------------------------------------- reductions
// Butterfly reductions over a full wavefront (64 lanes); every lane ends with
// the same value, combined in a fixed order (bit-reproducible).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace vdtq
