// Plain streaming passes for the benchmark's ceilings: each moves exactly
// the HBM bytes of one library launch and does no arithmetic beyond xor-ing
// its loads together (so no load can be dropped).  They are measuring
// instruments, not part of the library's C ABI (libvdtq_bench.so, loaded by
// bench.py only).
//
//   vdtq_bench_stream_rows: a [M][K] bf16 matrix read once, per 64-element
//     chunk `code_bytes` (32, 64 or 128) and `scale_bytes` (0, 2 or 4) bytes
//     written, plus `row_bytes` (0 or 4) per row: the traffic of a quantize
//     launch (NVFP4 32 + 4, INT8 64 + 4 per row, MXFP4 32 + 2, MXFP8 64 + 2,
//     BF16 128).
//   vdtq_bench_stream_3r1w: three bf16 vectors of n elements read, one
//     written: the traffic of block_stats with a bf16 delta cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

// One workgroup per 256 chunks; every load and store instruction of a wave
// covers consecutive 16-byte vectors.
__global__ __launch_bounds__(kThreads) void stream_rows_kernel(const uint4* __restrict__ x, int64_t chunks,
                                                               int cpr, int code_bytes, int scale_bytes,
                                                               int row_bytes, uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s, uint32_t* __restrict__ r) {
  const int64_t base = (int64_t)blockIdx.x * kThreads;     // first chunk of the workgroup
  const int64_t nvec = (chunks - base < kThreads ? chunks - base : kThreads) * 8;
  const int t = threadIdx.x;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t j = (int64_t)i * kThreads + t;
    v[i] = j < nvec ? x[base * 8 + j] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint4 a = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    a.x ^= v[i].x; a.y ^= v[i].y; a.z ^= v[i].z; a.w ^= v[i].w;
  }
  const int64_t c = base + t;
  uint4* qo = reinterpret_cast<uint4*>(q + base * code_bytes);
  const int per = code_bytes / 16;
  const int64_t nout = (chunks - base < kThreads ? chunks - base : kThreads) * per;
  for (int i = 0; i < per; ++i) {
    const int64_t j = (int64_t)i * kThreads + t;
    if (j < nout) qo[j] = make_uint4(a.x + i, a.y, a.z, a.w);
  }
  if (c >= chunks) return;
  if (scale_bytes == 4) reinterpret_cast<uint32_t*>(s)[c] = a.x ^ a.y;
  else if (scale_bytes == 2) reinterpret_cast<uint16_t*>(s)[c] = (uint16_t)(a.z ^ a.w);
  if (row_bytes && (c % cpr) == 0) r[c / cpr] = a.x ^ a.w;
}

__global__ __launch_bounds__(kThreads) void stream_3r1w_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                               const uint4* __restrict__ c, uint4* __restrict__ d,
                                                               int64_t vecs) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < vecs; i += stride) {
    const uint4 u = a[i], v = b[i], w = c[i];
    d[i] = make_uint4(u.x ^ v.x ^ w.x, u.y ^ v.y ^ w.y, u.z ^ v.z ^ w.z, u.w ^ v.w ^ w.w);
  }
}

}  // namespace

extern "C" {

// x: contiguous bf16 [M][K], K a multiple of 64, 16-byte aligned; q: M*K/64
// chunks of code_bytes; s: chunks of scale_bytes; r: M uint32 when
// row_bytes == 4.  Returns 0 or a hipError_t.
int vdtq_bench_stream_rows(const void* x, int64_t M, int64_t K, int code_bytes, int scale_bytes, int row_bytes,
                           void* q, void* s, void* r, void* stream) {
  if (M <= 0 || K <= 0 || K % 64 || (code_bytes != 32 && code_bytes != 64 && code_bytes != 128) ||
      (scale_bytes != 0 && scale_bytes != 2 && scale_bytes != 4) || (row_bytes != 0 && row_bytes != 4))
    return (int)hipErrorInvalidValue;
  const int64_t chunks = M * (K / 64);
  const unsigned grid = (unsigned)((chunks + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(stream_rows_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(x), chunks, (int)(K / 64), code_bytes, scale_bytes, row_bytes,
                     static_cast<uint8_t*>(q), static_cast<uint8_t*>(s), static_cast<uint32_t*>(r));
  return (int)hipGetLastError();
}

// a, b, c read, d written: n bf16 elements each, n a multiple of 8,
// 16-byte aligned.
int vdtq_bench_stream_3r1w(const void* a, const void* b, const void* c, void* d, int64_t n, void* stream) {
  if (n <= 0 || n % 8) return (int)hipErrorInvalidValue;
  const int64_t vecs = n / 8;
  int64_t grid = (vecs + 4 * kThreads - 1) / (4 * kThreads);   // 4 vectors per thread
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(stream_3r1w_kernel, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(a), static_cast<const uint4*>(b), static_cast<const uint4*>(c),
                     static_cast<uint4*>(d), vecs);
  return (int)hipGetLastError();
}

}  // extern "C"
