// C ABI of the library: argument validation, status codes, the thread-local
// error message, and dispatch to the kernel launchers.  Nothing is enqueued
// unless every argument checks out.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/vdtq.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return VDTQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VDTQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kI32 = 2147483647;

}  // namespace

extern "C" {

const char* vdtq_last_error(void) { return g_err.c_str(); }

const char* vdtq_version(void) { return "vdtq 0.1.0 gfx950"; }

size_t vdtq_workspace_bytes(int op, int64_t M, int64_t K) {
  if (op == VDTQ_OP_HADAMARD_QUANTIZE) return vdtq::hq_workspace_bytes(M, K);
  if (op == VDTQ_OP_BLOCK_STATS) return vdtq::bs_workspace_bytes(M);
  if (op == VDTQ_OP_QGEMM) return vdtq::qgemm_workspace_bytes(M, K);
  return 0;
}

}  // extern "C"

// Every check of hadamard_quantize's arguments except the workspace.
static int hq_check(const void* x_dev, int64_t M, int64_t K, int64_t ldx, int had_block, int fmt,
                    unsigned flags, void* q_dev, void* scales_dev, float* tensor_scale_dev, double* stats_dev) {
  if (M < 0 || M > kI32) return fail(VDTQ_EINVAL, "hadamard_quantize: M=%lld out of range", (long long)M);
  if (K <= 0 || K > kI32 || K % 16) return fail(VDTQ_EINVAL, "hadamard_quantize: K=%lld must be a positive multiple of 16", (long long)K);
  if (had_block != 16 && had_block != 32 && had_block != 64 && had_block != 128 && had_block != 256)
    return fail(VDTQ_EINVAL, "hadamard_quantize: had_block=%d must be 16, 32, 64, 128 or 256", had_block);
  if (K % had_block) return fail(VDTQ_EINVAL, "hadamard_quantize: K=%lld not a multiple of had_block=%d", (long long)K, had_block);
  if (ldx < K || ldx % 8) return fail(VDTQ_EINVAL, "hadamard_quantize: ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  if (fmt != VDTQ_FMT_NVFP4 && fmt != VDTQ_FMT_INT8 && fmt != VDTQ_FMT_BF16 && fmt != VDTQ_FMT_MXFP4 &&
      fmt != VDTQ_FMT_MXFP8)
    return fail(VDTQ_EINVAL, "hadamard_quantize: fmt=%d", fmt);
  if ((fmt == VDTQ_FMT_MXFP4 || fmt == VDTQ_FMT_MXFP8) && K % 32)
    return fail(VDTQ_EINVAL, "hadamard_quantize: MX formats need K=%lld to be a multiple of 32", (long long)K);
  if (flags & ~(VDTQ_AMAX_GIVEN | VDTQ_STATS | VDTQ_GELU)) return fail(VDTQ_EINVAL, "hadamard_quantize: unknown flags 0x%x", flags);
  if (fmt != VDTQ_FMT_NVFP4 && (flags & VDTQ_AMAX_GIVEN))
    return fail(VDTQ_EINVAL, "hadamard_quantize: VDTQ_AMAX_GIVEN applies to NVFP4 only");
  if (fmt == VDTQ_FMT_INT8 && K > 16384)
    return fail(VDTQ_EUNSUPPORTED, "hadamard_quantize: INT8 rows longer than 16384 (K=%lld)", (long long)K);
  const int64_t cpr = (K + 63) / 64;
  if (M * cpr > kI32) return fail(VDTQ_EINVAL, "hadamard_quantize: M*ceil(K/64) exceeds 2^31");
  if (M > 0) {
    if (!x_dev || !q_dev || (fmt != VDTQ_FMT_BF16 && !scales_dev))
      return fail(VDTQ_EINVAL, "hadamard_quantize: null x/q/scales");
    if (!aligned(x_dev, 16) || !aligned(q_dev, 16) || (fmt != VDTQ_FMT_BF16 && !aligned(scales_dev, 4)))
      return fail(VDTQ_EINVAL, "hadamard_quantize: x and q must be 16-byte aligned, scales 4-byte aligned");
  }
  if (fmt == VDTQ_FMT_NVFP4 && (!tensor_scale_dev || !aligned(tensor_scale_dev, 4)))
    return fail(VDTQ_EINVAL, "hadamard_quantize: NVFP4 needs an aligned tensor_scale (float[2])");
  if ((flags & VDTQ_STATS) && (!stats_dev || !aligned(stats_dev, 8)))
    return fail(VDTQ_EINVAL, "hadamard_quantize: VDTQ_STATS needs an aligned stats buffer (double[4])");
  return VDTQ_OK;
}

extern "C" {

int hadamard_quantize(const void* x_dev, int64_t M, int64_t K, int64_t ldx, int had_block, int fmt,
                      unsigned flags, void* q_dev, void* scales_dev, float* tensor_scale_dev,
                      double* stats_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  const int rc = hq_check(x_dev, M, K, ldx, had_block, fmt, flags, q_dev, scales_dev, tensor_scale_dev, stats_dev);
  if (rc != VDTQ_OK) return rc;
  const bool need_ws = (flags & VDTQ_STATS) || (fmt == VDTQ_FMT_NVFP4 && !(flags & VDTQ_AMAX_GIVEN));
  if (need_ws) {
    const size_t need = vdtq::hq_workspace_bytes(M, K);
    if (!ws_dev || !aligned(ws_dev, 16) || ws_bytes < need)
      return fail(VDTQ_EINVAL, "hadamard_quantize: workspace of %zu bytes (16-byte aligned) required, got %zu", need, ws_bytes);
  }
  hipError_t e = vdtq::launch_hadamard_quantize(x_dev, M, K, ldx, had_block, fmt, flags, q_dev, scales_dev,
                                                tensor_scale_dev, stats_dev, ws_dev,
                                                static_cast<hipStream_t>(stream));
  return hip_status(e, "hadamard_quantize launch");
}

int hadamard_quantize_noalloc(const void* x_dev, int64_t M, int64_t K, int64_t ldx, int had_block, int fmt,
                              unsigned flags, void* q_dev, void* scales_dev, float* tensor_scale_dev,
                              double* stats_dev, void* stream) {
  const int rc = hq_check(x_dev, M, K, ldx, had_block, fmt, flags, q_dev, scales_dev, tensor_scale_dev, stats_dev);
  if (rc != VDTQ_OK) return rc;
  const size_t need = vdtq::hq_workspace_bytes(M, K);
  if (need > VDTQ_NOALLOC_SCRATCH_BYTES)
    return fail(VDTQ_EUNSUPPORTED,
                "hadamard_quantize_noalloc: M=%lld K=%lld needs %zu bytes of scratch, above the %zu-byte maximum",
                (long long)M, (long long)K, need, (size_t)VDTQ_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  hipError_t e = vdtq::hq_noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "hadamard_quantize_noalloc: scratch address");
  e = vdtq::launch_hadamard_quantize(x_dev, M, K, ldx, had_block, fmt, flags, q_dev, scales_dev, tensor_scale_dev,
                                     stats_dev, scratch, static_cast<hipStream_t>(stream));
  return hip_status(e, "hadamard_quantize_noalloc launch");
}

static int qgemm_check(const char* name, const void* a_q, const void* a_s, const void* w_q, const void* w_s,
                       const float* w_ts, const float* bias, void* y, int64_t ldy, int out_dtype, int64_t M,
                       int64_t N, int64_t K) {
  if (M < 0 || M > kI32 || N < 0 || N > kI32) return fail(VDTQ_EINVAL, "%s: M=%lld N=%lld out of range", name, (long long)M, (long long)N);
  if (K <= 0 || K > kI32 || K % 16) return fail(VDTQ_EINVAL, "%s: K=%lld must be a positive multiple of 16", name, (long long)K);
  if (out_dtype != VDTQ_OUT_BF16 && out_dtype != VDTQ_OUT_F32) return fail(VDTQ_EINVAL, "%s: out_dtype=%d", name, out_dtype);
  if (ldy < N) return fail(VDTQ_EINVAL, "%s: ldy=%lld < N=%lld", name, (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return VDTQ_OK;
  if (!a_q || !a_s || !w_q || !w_s || !w_ts || !y) return fail(VDTQ_EINVAL, "%s: null pointer argument", name);
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(w_s, 8) || !aligned(w_ts, 4) ||
      !aligned(y, out_dtype ? 4 : 2) || (bias && !aligned(bias, 4)))
    return fail(VDTQ_EINVAL, "%s: misaligned pointer (codes need 16 bytes, scales 8)", name);
  if (((M + 255) / 256) * ((N + 255) / 256) > kI32)
    return fail(VDTQ_EUNSUPPORTED, "%s: too many output tiles", name);
  return VDTQ_OK;
}

static int qgemm_ws_check(const char* name, int64_t M, int64_t N, const void* ws, size_t ws_bytes) {
  if (M == 0 || N == 0) return VDTQ_OK;
  const size_t need = vdtq::qgemm_workspace_bytes(M, N);
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(VDTQ_EINVAL, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", name, need, ws_bytes);
  return VDTQ_OK;
}

int qgemm_w4a4(const uint8_t* a_q_dev, const uint8_t* a_s_dev, const float* a_ts_dev, const uint8_t* w_q_dev,
               const uint8_t* w_s_dev, const float* w_ts_dev, const float* bias_dev, void* y_dev, int64_t ldy,
               int out_dtype, int64_t M, int64_t N, int64_t K, void* ws_dev, size_t ws_bytes, void* stream) {
  int rc = qgemm_check("qgemm_w4a4", a_q_dev, a_s_dev, w_q_dev, w_s_dev, w_ts_dev, bias_dev, y_dev, ldy,
                       out_dtype, M, N, K);
  if (rc) return rc;
  if (M > 0 && N > 0 && (!a_ts_dev || !aligned(a_ts_dev, 4) || !aligned(a_s_dev, 8)))
    return fail(VDTQ_EINVAL, "qgemm_w4a4: null or misaligned a_ts / a_s");
  rc = qgemm_ws_check("qgemm_w4a4", M, N, ws_dev, ws_bytes);
  if (rc) return rc;
  hipError_t e = vdtq::launch_qgemm(0, a_q_dev, a_s_dev, a_ts_dev, w_q_dev, w_s_dev, w_ts_dev, bias_dev, y_dev,
                                    ldy, out_dtype, M, N, K, ws_dev, static_cast<hipStream_t>(stream));
  return hip_status(e, "qgemm_w4a4 launch");
}

int qgemm_w4a8(const int8_t* a_q_dev, const float* a_s_dev, const uint8_t* w_q_dev, const uint8_t* w_s_dev,
               const float* w_ts_dev, const float* bias_dev, void* y_dev, int64_t ldy, int out_dtype, int64_t M,
               int64_t N, int64_t K, void* ws_dev, size_t ws_bytes, void* stream) {
  int rc = qgemm_check("qgemm_w4a8", a_q_dev, a_s_dev, w_q_dev, w_s_dev, w_ts_dev, bias_dev, y_dev, ldy,
                       out_dtype, M, N, K);
  if (rc) return rc;
  if (M > 0 && N > 0 && !aligned(a_s_dev, 4)) return fail(VDTQ_EINVAL, "qgemm_w4a8: misaligned a_s");
  rc = qgemm_ws_check("qgemm_w4a8", M, N, ws_dev, ws_bytes);
  if (rc) return rc;
  hipError_t e = vdtq::launch_qgemm(1, a_q_dev, a_s_dev, nullptr, w_q_dev, w_s_dev, w_ts_dev, bias_dev, y_dev,
                                    ldy, out_dtype, M, N, K, ws_dev, static_cast<hipStream_t>(stream));
  return hip_status(e, "qgemm_w4a8 launch");
}

int qgemm_w4a16(const void* a_dev, const uint8_t* w_q_dev, const uint8_t* w_s_dev, const float* w_ts_dev,
                const float* bias_dev, void* y_dev, int64_t ldy, int out_dtype, int64_t M, int64_t N, int64_t K,
                void* ws_dev, size_t ws_bytes, void* stream) {
  const char* name = "qgemm_w4a16";
  if (M < 0 || M > kI32 || N < 0 || N > kI32) return fail(VDTQ_EINVAL, "%s: M=%lld N=%lld out of range", name, (long long)M, (long long)N);
  if (K <= 0 || K > kI32 || K % 16) return fail(VDTQ_EINVAL, "%s: K=%lld must be a positive multiple of 16", name, (long long)K);
  if (out_dtype != VDTQ_OUT_BF16 && out_dtype != VDTQ_OUT_F32) return fail(VDTQ_EINVAL, "%s: out_dtype=%d", name, out_dtype);
  if (ldy < N) return fail(VDTQ_EINVAL, "%s: ldy=%lld < N=%lld", name, (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!a_dev || !w_q_dev || !w_s_dev || !w_ts_dev || !y_dev) return fail(VDTQ_EINVAL, "%s: null pointer argument", name);
  if (!aligned(a_dev, 16) || !aligned(w_q_dev, 16) || !aligned(w_s_dev, 4) || !aligned(w_ts_dev, 4) ||
      !aligned(y_dev, out_dtype ? 4 : 2) || (bias_dev && !aligned(bias_dev, 4)))
    return fail(VDTQ_EINVAL, "%s: misaligned pointer (a and codes need 16 bytes, scales 4)", name);
  if (K % 64) return fail(VDTQ_EUNSUPPORTED, "%s: K=%lld is not a multiple of 64", name, (long long)K);
  if (M * K * 2 >= (int64_t(1) << 32) || N * K / 2 >= (int64_t(1) << 32))
    return fail(VDTQ_EUNSUPPORTED, "%s: operands of 4 GB or more", name);
  if (((M + 255) / 256) * ((N + 255) / 256) > kI32) return fail(VDTQ_EUNSUPPORTED, "%s: too many output tiles", name);
  const int rc = qgemm_ws_check(name, M, N, ws_dev, ws_bytes);
  if (rc != VDTQ_OK) return rc;
  hipError_t e = vdtq::launch_qgemm_w4a16(a_dev, w_q_dev, w_s_dev, w_ts_dev, bias_dev, y_dev, ldy, out_dtype, M, N,
                                          K, ws_dev, static_cast<hipStream_t>(stream));
  return hip_status(e, "qgemm_w4a16 launch");
}

int qgemm_mx(int a_fmt, const uint8_t* a_q_dev, const uint8_t* a_s_dev, const uint8_t* w_q_dev,
             const uint8_t* w_s_dev, const float* bias_dev, void* y_dev, int64_t ldy, int out_dtype, int64_t M,
             int64_t N, int64_t K, void* ws_dev, size_t ws_bytes, void* stream) {
  const char* name = "qgemm_mx";
  if (a_fmt != VDTQ_FMT_MXFP4 && a_fmt != VDTQ_FMT_MXFP8) return fail(VDTQ_EINVAL, "%s: a_fmt=%d", name, a_fmt);
  if (M < 0 || M > kI32 || N < 0 || N > kI32) return fail(VDTQ_EINVAL, "%s: M=%lld N=%lld out of range", name, (long long)M, (long long)N);
  if (K <= 0 || K > kI32 || K % 32) return fail(VDTQ_EINVAL, "%s: K=%lld must be a positive multiple of 32", name, (long long)K);
  if (out_dtype != VDTQ_OUT_BF16 && out_dtype != VDTQ_OUT_F32) return fail(VDTQ_EINVAL, "%s: out_dtype=%d", name, out_dtype);
  if (ldy < N) return fail(VDTQ_EINVAL, "%s: ldy=%lld < N=%lld", name, (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!a_q_dev || !a_s_dev || !w_q_dev || !w_s_dev || !y_dev) return fail(VDTQ_EINVAL, "%s: null pointer argument", name);
  if (!aligned(a_q_dev, 16) || !aligned(w_q_dev, 16) || !aligned(a_s_dev, 4) || !aligned(w_s_dev, 4) ||
      !aligned(y_dev, out_dtype ? 4 : 2) || (bias_dev && !aligned(bias_dev, 4)))
    return fail(VDTQ_EINVAL, "%s: misaligned pointer (codes need 16 bytes, scales 4)", name);
  if (K % 128) return fail(VDTQ_EUNSUPPORTED, "%s: K=%lld is not a multiple of 128", name, (long long)K);
  const bool a8 = a_fmt == VDTQ_FMT_MXFP8;
  if ((a8 ? M * K : M * K / 2) >= (int64_t(1) << 32) || N * K / 2 >= (int64_t(1) << 32))
    return fail(VDTQ_EUNSUPPORTED, "%s: operands of 4 GB or more", name);
  if (((M + 255) / 256) * ((N + 255) / 256) > kI32) return fail(VDTQ_EUNSUPPORTED, "%s: too many output tiles", name);
  int rc = qgemm_ws_check(name, M, N, ws_dev, ws_bytes);
  if (rc) return rc;
  hipError_t e = vdtq::launch_qgemm_mx(a8, a_q_dev, a_s_dev, w_q_dev, w_s_dev, bias_dev, y_dev, ldy, out_dtype, M,
                                       N, K, ws_dev, static_cast<hipStream_t>(stream));
  return hip_status(e, "qgemm_mx launch");
}

int qgemm_mx_quant(int a_fmt, const uint8_t* a_q_dev, const uint8_t* a_s_dev, const uint8_t* w_q_dev,
                   const uint8_t* w_s_dev, const float* bias_dev, int had_block, int out_fmt, unsigned flags,
                   uint8_t* q_out_dev, uint8_t* s_out_dev, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* name = "qgemm_mx_quant";
  if (a_fmt != VDTQ_FMT_MXFP4 && a_fmt != VDTQ_FMT_MXFP8) return fail(VDTQ_EINVAL, "%s: a_fmt=%d", name, a_fmt);
  if (out_fmt != VDTQ_FMT_MXFP4 && out_fmt != VDTQ_FMT_MXFP8) return fail(VDTQ_EINVAL, "%s: out_fmt=%d", name, out_fmt);
  if (flags & ~VDTQ_GELU) return fail(VDTQ_EINVAL, "%s: unknown flags 0x%x", name, flags);
  if (had_block != 64) return fail(VDTQ_EUNSUPPORTED, "%s: had_block=%d (only 64)", name, had_block);
  if (M < 0 || M > kI32 || N < 0 || N > kI32) return fail(VDTQ_EINVAL, "%s: M=%lld N=%lld out of range", name, (long long)M, (long long)N);
  if (N % 64) return fail(VDTQ_EINVAL, "%s: N=%lld not a multiple of had_block=64", name, (long long)N);
  if (K <= 0 || K > kI32 || K % 32) return fail(VDTQ_EINVAL, "%s: K=%lld must be a positive multiple of 32", name, (long long)K);
  if (M == 0 || N == 0) return ok();
  if (!a_q_dev || !a_s_dev || !w_q_dev || !w_s_dev || !q_out_dev || !s_out_dev)
    return fail(VDTQ_EINVAL, "%s: null pointer argument", name);
  if (!aligned(a_q_dev, 16) || !aligned(w_q_dev, 16) || !aligned(q_out_dev, 16) || !aligned(a_s_dev, 4) ||
      !aligned(w_s_dev, 4) || !aligned(s_out_dev, 4) || (bias_dev && !aligned(bias_dev, 16)))
    return fail(VDTQ_EINVAL, "%s: misaligned pointer (codes and bias need 16 bytes, scales 4)", name);
  if (K % 128) return fail(VDTQ_EUNSUPPORTED, "%s: K=%lld is not a multiple of 128", name, (long long)K);
  const bool a8 = a_fmt == VDTQ_FMT_MXFP8;
  if ((a8 ? M * K : M * K / 2) >= (int64_t(1) << 32) || N * K / 2 >= (int64_t(1) << 32))
    return fail(VDTQ_EUNSUPPORTED, "%s: operands of 4 GB or more", name);
  if (((M + 255) / 256) * ((N + 255) / 256) > kI32) return fail(VDTQ_EUNSUPPORTED, "%s: too many output tiles", name);
  hipError_t e = vdtq::launch_qgemm_mx_quant(a8, a_q_dev, a_s_dev, w_q_dev, w_s_dev, bias_dev,
                                             out_fmt == VDTQ_FMT_MXFP8, (flags & VDTQ_GELU) != 0, q_out_dev,
                                             s_out_dev, M, N, K, static_cast<hipStream_t>(stream));
  return hip_status(e, "qgemm_mx_quant launch");
}

int block_stats(const void* in_dev, const void* out_dev, const void* dprev_dev, void* dnew_dev, int64_t n,
                double* stats_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  if (n < 0) return fail(VDTQ_EINVAL, "block_stats: n=%lld < 0", (long long)n);
  if (!stats_dev || !aligned(stats_dev, 8)) return fail(VDTQ_EINVAL, "block_stats: null or misaligned stats");
  if (n > 0 && (!in_dev || !out_dev)) return fail(VDTQ_EINVAL, "block_stats: null in/out");
  if (!aligned(in_dev, 16) || !aligned(out_dev, 16) || !aligned(dprev_dev, 16) || !aligned(dnew_dev, 16))
    return fail(VDTQ_EINVAL, "block_stats: bf16 buffers must be 16-byte aligned");
  if (dnew_dev && dnew_dev == dprev_dev) return fail(VDTQ_EINVAL, "block_stats: dnew must not alias dprev");
  const size_t need = vdtq::bs_workspace_bytes(n);
  if (!ws_dev || !aligned(ws_dev, 16) || ws_bytes < need)
    return fail(VDTQ_EINVAL, "block_stats: workspace of %zu bytes (16-byte aligned) required, got %zu", need, ws_bytes);
  hipError_t e = vdtq::launch_block_stats(in_dev, out_dev, dprev_dev, dnew_dev, n, stats_dev, ws_dev,
                                          static_cast<hipStream_t>(stream));
  return hip_status(e, "block_stats launch");
}

int block_stats_mx8(const void* in_dev, const void* out_dev, const uint8_t* dprev_q_dev, const uint8_t* dprev_s_dev,
                    uint8_t* dnew_q_dev, uint8_t* dnew_s_dev, int64_t n, double* stats_dev, void* ws_dev,
                    size_t ws_bytes, void* stream) {
  const char* name = "block_stats_mx8";
  if (n < 0 || n % 32) return fail(VDTQ_EINVAL, "%s: n=%lld must be a non-negative multiple of 32", name, (long long)n);
  if (!stats_dev || !aligned(stats_dev, 8)) return fail(VDTQ_EINVAL, "%s: null or misaligned stats", name);
  if ((dprev_q_dev == nullptr) != (dprev_s_dev == nullptr) || (dnew_q_dev == nullptr) != (dnew_s_dev == nullptr))
    return fail(VDTQ_EINVAL, "%s: codes and scales of a delta are given together or not at all", name);
  if (n > 0 && (!in_dev || !out_dev)) return fail(VDTQ_EINVAL, "%s: null in/out", name);
  if (!aligned(in_dev, 16) || !aligned(out_dev, 16) || !aligned(dprev_q_dev, 8) || !aligned(dnew_q_dev, 8))
    return fail(VDTQ_EINVAL, "%s: in/out must be 16-byte aligned, delta codes 8-byte aligned", name);
  if (dnew_q_dev && (dnew_q_dev == dprev_q_dev || dnew_s_dev == dprev_s_dev))
    return fail(VDTQ_EINVAL, "%s: dnew must not alias dprev", name);
  const size_t need = vdtq::bs_workspace_bytes(n);
  if (!ws_dev || !aligned(ws_dev, 16) || ws_bytes < need)
    return fail(VDTQ_EINVAL, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", name, need, ws_bytes);
  hipError_t e = vdtq::launch_block_stats_mx8(in_dev, out_dev, dprev_q_dev, dprev_s_dev, dnew_q_dev, dnew_s_dev, n,
                                              stats_dev, ws_dev, static_cast<hipStream_t>(stream));
  return hip_status(e, "block_stats_mx8 launch");
}

}  // extern "C"
