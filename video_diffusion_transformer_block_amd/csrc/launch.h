// Host-side launchers of the gfx950 kernels (one per translation unit); the
// C ABI in api.cpp validates every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vdtq {

// Compute units of the current device, cached per device; `fallback` when
// the query fails.
inline int device_cu_count(int fallback = 256) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fallback;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t hq_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_hadamard_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, int b, int fmt,
                                    unsigned flags, void* q, void* scales, float* ts,
                                    double* stats, void* ws, hipStream_t st);

// Device address of this GPU's allocation-free scratch array
// (VDTQ_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up once per device.
hipError_t hq_noalloc_scratch(void** ptr);

// Device address of this GPU's GELU lookup table (hadamard_common.h), built
// on `st` by the first call on the device, which then waits for it; a call
// on a capturing stream records the build instead and leaves it to be done
// again by the next call outside capture.
hipError_t gelu_table(hipStream_t st, const uint16_t** tab);

size_t qgemm_workspace_bytes(int64_t M, int64_t N);
hipError_t launch_qgemm(int afmt, const void* a_q, const void* a_s, const float* a_ts,
                        const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                        const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                        int64_t N, int64_t K, void* ws, hipStream_t st);

hipError_t launch_qgemm_w4a16(const void* a, const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M, int64_t N,
                              int64_t K, void* ws, hipStream_t st);

hipError_t launch_qgemm_mx(bool a_fp8, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                           const uint8_t* w_s, const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                           int64_t N, int64_t K, void* ws, hipStream_t st);

hipError_t launch_qgemm_mx_quant(bool a_fp8, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                                 const uint8_t* w_s, const float* bias, bool out_fp8, bool gelu, uint8_t* q_out,
                                 uint8_t* s_out, int64_t M, int64_t N, int64_t K, hipStream_t st);

size_t bs_workspace_bytes(int64_t n);
hipError_t launch_block_stats(const void* in, const void* out, const void* dprev, void* dnew,
                              int64_t n, double* stats, void* ws, hipStream_t st);
hipError_t launch_block_stats_mx8(const void* in, const void* out, const uint8_t* dprev_q, const uint8_t* dprev_s,
                                  uint8_t* dnew_q, uint8_t* dnew_s, int64_t n, double* stats, void* ws,
                                  hipStream_t st);

}  // namespace vdtq
