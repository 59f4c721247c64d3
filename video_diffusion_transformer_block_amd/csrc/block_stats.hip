// block_stats: one pass over a transformer block's input, output and cached
// residual delta (gfx950).
//
// The operation: gist.science "6Bit-Diffusion: Inference-Time Mixed-Precision
// Quantization for Video Diffusion Models" §2.A (Gamma_{t-1}, the block's
// relative input-output difference, picks the precision), §2.B (the
// similarity of Delta_{t-1} and Delta_{t-2} predicts a skip; Delta is cached)
// and youleyou.com article §三 (max/mean outlier ratio) and §七 (these online
// metrics are an extra pass whose cost must stay small).
//
// HBM-bound: 8 bytes per element (in, out, Delta_prev read; Delta_new
// written).  Each thread handles 4 x 8 elements per step with 16-byte
// buffer accesses (all twelve loads in flight at once) in a grid-stride loop
// over a grid sized from n only (at most 1024 workgroups), accumulates in
// fp64, and the workgroup and grid reductions run in a fixed order: the
// eight results are bit-identical from run to run.  The grid reduction is
// done by the last workgroup to finish (no second launch).
//
// block_stats_mx8_kernel is the same pass with the delta cache in MXFP8
// (youleyou.com article §七: the cache's memory can be cut by storing it in
// low precision): Delta_new = MXFP8(out - in) (E4M3 elements, one E8M0
// exponent per 32 consecutive elements, the OCP Microscaling conversion)
// and Delta_prev read as MXFP8, so a step moves 6 + 1/16 bytes per element
// instead of 8.  Four consecutive lanes hold one 32-element block (8
// elements each), combine its maximum with two lane exchanges, and write 32
// contiguous code bytes.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace vdtq {

constexpr int BS_THREADS = 256;
constexpr int BS_UNROLL = 4;                     // 16-byte vectors per thread and step (bf16 pass)
constexpr int BS_STEPS = 2;                      // steps per workgroup (fewer partials to combine)
#ifndef VDTQ_BS_GRID_BF16
#define VDTQ_BS_GRID_BF16 1024
#endif
constexpr int BS_GRID_BF16 = VDTQ_BS_GRID_BF16;  // grid cap of the bf16-cache pass
constexpr int BS_GRID_MX8 = 2048;                // grid cap of the MXFP8-cache pass (one vector per step)
constexpr int BS_HEADER = 256;                   // workspace bytes before the partials (completion counter)

// Workgroups of a launch: per_thread vectors for each of its threads, at
// most `cap` (the loops are grid-stride); the bf16 pass takes BS_STEPS
// steps of BS_UNROLL vectors per thread, the MXFP8 pass one vector.
static int bs_grid(int64_t n, int per_thread = BS_UNROLL * BS_STEPS, int cap = BS_GRID_BF16) {
  const int64_t vecs = (n + 7) / 8, per_wg = (int64_t)BS_THREADS * per_thread;
  int64_t g = (vecs + per_wg - 1) / per_wg;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}
static int bs_grid_mx8(int64_t n) { return bs_grid(n, 4, BS_GRID_MX8); }   // >= 4 vectors per thread

struct Acc8 {
  double d2 = 0, i2 = 0, dd2 = 0, p2 = 0, si = 0, so = 0;
  float mi = 0.0f, mo = 0.0f;
};

// The squares of fp32 and bf16 values are exact in fp64, so each fma below
// rounds once, as the separate product and sum would.
template <bool HAS_PREV>
__device__ __forceinline__ void acc_one(Acc8& a, float xi, float xo, float dp, uint32_t& dnew_bits) {
  const float d = xo - xi;                       // fp32 RN
  dnew_bits = f32_to_bf16_bits(d);
  const double dd = (double)d, ii = (double)xi;
  a.d2 = fma(dd, dd, a.d2);
  a.i2 = fma(ii, ii, a.i2);
  if (HAS_PREV) {
    const double dn = (double)__uint_as_float(dnew_bits << 16);
    const double pp = (double)dp;
    const double df = dn - pp;                   // fp64 RN
    a.dd2 += df * df;
    a.p2 = fma(pp, pp, a.p2);
  }
  const float ai = fabsf(xi), ao = fabsf(xo);
  a.mi = fmaxf(a.mi, ai);
  a.mo = fmaxf(a.mo, ao);
  a.si += fabs(ii);
  a.so += (double)ao;
}

// End of a statistics workgroup: its eight partials (fixed-order workgroup
// reduction) go to part[k * MAX_GRID + wg], k = 0..7, with agent-scope
// stores, which write through to the point where every XCD sees them; once
// they are complete, one lane counts the workgroup in.  The workgroup that
// finds itself last reduces the partials of the whole grid: for each k,
// thread t takes partials t, t + 256, ... in order (consecutive lanes read
// consecutive doubles), then the waves are combined in order, so the sums
// are the same whichever workgroup is last and the results are
// bit-identical from run to run.  It writes the eight statistics and sets
// the counter back to zero for the next call.  MAX_GRID bounds the grid.
template <int MAX_GRID>
__device__ __forceinline__ void bs_finish(const Acc8& a, double* part, unsigned* counter, double* stats) {
  __shared__ double red[8][BS_THREADS / 64];
  __shared__ int last;
  double vals[8] = {a.d2, a.i2, a.dd2, a.p2, (double)a.mi, a.si, (double)a.mo, a.so};
#pragma unroll
  for (int k = 0; k < 8; ++k) vals[k] = (k == 4 || k == 6) ? wave_max_d(vals[k]) : wave_sum(vals[k]);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < 8; ++k) red[k][w] = vals[k];
  __syncthreads();
  if (threadIdx.x < 8) {
    const int k = threadIdx.x;
    double r = red[k][0];
    for (int i = 1; i < BS_THREADS / 64; ++i) r = (k == 4 || k == 6) ? fmax(r, red[k][i]) : r + red[k][i];
    __hip_atomic_store(part + k * MAX_GRID + blockIdx.x, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);                 // the partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  // every load of the tail is issued before the first is used (addresses
  // clamped into the grid, values past it replaced by zeros, which change
  // no sum or maximum)
  constexpr int PU = (MAX_GRID + BS_THREADS - 1) / BS_THREADS;
  const int np = (int)gridDim.x;
  double q[PU][8];
#pragma unroll
  for (int u = 0; u < PU; ++u) {
    const int i = min((int)threadIdx.x + BS_THREADS * u, np - 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) q[u][k] = __hip_atomic_load(part + k * MAX_GRID + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) vals[k] = 0.0;
#pragma unroll
  for (int u = 0; u < PU; ++u) {
    const bool in = (int)threadIdx.x + BS_THREADS * u < np;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double x = in ? q[u][k] : 0.0;
      vals[k] = (k == 4 || k == 6) ? fmax(vals[k], x) : vals[k] + x;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) vals[k] = (k == 4 || k == 6) ? wave_max_d(vals[k]) : wave_sum(vals[k]);
  __syncthreads();                               // red[] is reused
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < 8; ++k) red[k][w] = vals[k];
  __syncthreads();
  if (threadIdx.x < 8) {
    const int k = threadIdx.x;
    double r = red[k][0];
    for (int i = 1; i < BS_THREADS / 64; ++i) r = (k == 4 || k == 6) ? fmax(r, red[k][i]) : r + red[k][i];
    stats[k] = r;
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool HAS_PREV>
__global__ __launch_bounds__(BS_THREADS) void block_stats_kernel(const uint16_t* in, const uint16_t* out,
                                                                 const uint16_t* dprev, uint16_t* dnew,
                                                                 int64_t n, double* part, unsigned* counter,
                                                                 double* stats) {
  Acc8 a;
  const int64_t nvec = n / 8;
  // Each step covers BS_UNROLL * BS_THREADS consecutive vectors through
  // buffer resources bounded at the end of the data: every load of the step
  // is issued before the first is used, vectors past the end read as zeros
  // (which add nothing to any sum or maximum) and their stores are dropped.
  // An absent Delta_prev or Delta_new gets an empty resource.
  constexpr int kSpan = BS_THREADS * BS_UNROLL;
  const int64_t step = (int64_t)gridDim.x * kSpan;
  const uint32_t lane = threadIdx.x * 16u;
  for (int64_t vb = (int64_t)blockIdx.x * kSpan; vb < nvec; vb += step) {
    const uint32_t bytes = (uint32_t)min<int64_t>(nvec - vb, kSpan) * 16u;
    const __amdgpu_buffer_rsrc_t ri = raw_buffer(in + vb * 8, bytes);
    const __amdgpu_buffer_rsrc_t ro = raw_buffer(out + vb * 8, bytes);
    const __amdgpu_buffer_rsrc_t rp = raw_buffer(HAS_PREV ? dprev + vb * 8 : in, HAS_PREV ? bytes : 0u);
    const __amdgpu_buffer_rsrc_t rn = raw_buffer(dnew ? dnew + vb * 8 : in, dnew ? bytes : 0u);
    uint4 wi[BS_UNROLL], wo[BS_UNROLL], wp[BS_UNROLL];
#pragma unroll
    for (int u = 0; u < BS_UNROLL; ++u) {
      wi[u] = buffer_load16(ri, lane + u * BS_THREADS * 16);
      wo[u] = buffer_load16(ro, lane + u * BS_THREADS * 16);
      wp[u] = buffer_load16(rp, lane + u * BS_THREADS * 16);
    }
#pragma unroll
    for (int u = 0; u < BS_UNROLL; ++u) {
      const uint32_t ii[4] = {wi[u].x, wi[u].y, wi[u].z, wi[u].w};
      const uint32_t oo[4] = {wo[u].x, wo[u].y, wo[u].z, wo[u].w};
      const uint32_t pp[4] = {wp[u].x, wp[u].y, wp[u].z, wp[u].w};
      uint32_t res[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t b0, b1;
        acc_one<HAS_PREV>(a, bf16_lo(ii[k]), bf16_lo(oo[k]), bf16_lo(pp[k]), b0);
        acc_one<HAS_PREV>(a, bf16_hi(ii[k]), bf16_hi(oo[k]), bf16_hi(pp[k]), b1);
        res[k] = b0 | (b1 << 16);
      }
      buffer_store16(rn, lane + u * BS_THREADS * 16, make_uint4(res[0], res[1], res[2], res[3]));
    }
  }
  // scalar tail (n % 8 elements), taken by the first workgroup's first lanes
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t i = nvec * 8 + threadIdx.x;
    uint32_t b;
    const float pv = HAS_PREV ? __uint_as_float((uint32_t)dprev[i] << 16) : 0.0f;
    acc_one<HAS_PREV>(a, __uint_as_float((uint32_t)in[i] << 16), __uint_as_float((uint32_t)out[i] << 16), pv, b);
    if (dnew) dnew[i] = (uint16_t)b;
  }
  bs_finish<BS_GRID_BF16>(a, part, counter, stats);
}

// 2^e as fp64 (e in [-127, 127])
__device__ __forceinline__ double exp2d(int e) { return __longlong_as_double((long long)(e + 1023) << 52); }

// The E4M3 value of each byte of w (hardware conversion, exact), times 2^e.
__device__ __forceinline__ void fp8x4_values(uint32_t w, int e, double (&v)[4]) {
  const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const float2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  const double s = exp2d(e);
  v[0] = (double)lo[0] * s; v[1] = (double)lo[1] * s; v[2] = (double)hi[0] * s; v[3] = (double)hi[1] * s;
}

// One 16-byte vector (8 elements) of the MXFP8 pass: statistics, the block
// maximum over the vector's four lanes (lanes 4k .. 4k + 3 hold one
// 32-element block and run this together), the E8M0 exponent, the E4M3
// codes, and the similarity terms against the previous cached delta.
__device__ __forceinline__ void mx8_vector(Acc8& a, const uint4& wi, const uint4& wo, bool has_prev, uint2 pq,
                                           int ep, uint32_t (&codes)[2], int& e) {
  const uint32_t ii[4] = {wi.x, wi.y, wi.z, wi.w};
  const uint32_t oo[4] = {wo.x, wo.y, wo.z, wo.w};
  float d[8];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float i0 = bf16_lo(ii[k]), i1 = bf16_hi(ii[k]), o0 = bf16_lo(oo[k]), o1 = bf16_hi(oo[k]);
    d[2 * k] = o0 - i0;                           // fp32 RN
    d[2 * k + 1] = o1 - i1;
    const float e0[2] = {i0, i1}, e1[2] = {o0, o1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const double dd = (double)d[2 * k + q], xi = (double)e0[q];
      a.d2 += dd * dd;
      a.i2 += xi * xi;
      const float ai = fabsf(e0[q]), ao = fabsf(e1[q]);
      a.mi = fmaxf(a.mi, ai);
      a.mo = fmaxf(a.mo, ao);
      a.si += (double)ai;
      a.so += (double)ao;
    }
    amax = fmaxf(amax, fmaxf(fabsf(d[2 * k]), fabsf(d[2 * k + 1])));
  }
  // the block's maximum over its four lanes (all active together)
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  // E8M0 exponent: floor(log2 amax) - 8 clamped to [-127, 127]; zero and
  // fp32-subnormal maxima give -127
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  e = ex == 0 ? -127 : min(max(ex - 127 - 8, -127), 127);
  // d * 2^-e as two exact power-of-two factors (normal fp32 each); clamp
  // to +-448 (the conversion itself does not saturate)
  const int n1 = -e / 2, n2 = -e - n1;
  const float m1 = __uint_as_float((uint32_t)(n1 + 127) << 23), m2 = __uint_as_float((uint32_t)(n2 + 127) << 23);
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = __builtin_amdgcn_fmed3f((d[4 * w + i] * m1) * m2, -448.0f, 448.0f);
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], x, true);
    codes[w] = (uint32_t)x;
  }
  if (has_prev) {
    const uint32_t pw[2] = {pq.x, pq.y};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      double dn[4], dp[4];
      fp8x4_values(codes[w], e, dn);
      fp8x4_values(pw[w], ep, dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double df = dn[i] - dp[i];
        a.dd2 += df * df;
        a.p2 += dp[i] * dp[i];
      }
    }
  }
}

__global__ __launch_bounds__(BS_THREADS) void block_stats_mx8_kernel(const uint16_t* in, const uint16_t* out,
                                                                     const uint8_t* dprev_q, const uint8_t* dprev_s,
                                                                     uint8_t* dnew_q, uint8_t* dnew_s, int64_t n,
                                                                     double* part, unsigned* counter,
                                                                     double* stats) {
  Acc8 a;
  const bool has_prev = dprev_q != nullptr;
  const int64_t nvec = n / 8;                    // a multiple of 4: n % 32 == 0
  const int64_t stride = (int64_t)gridDim.x * BS_THREADS;
  for (int64_t v = (int64_t)blockIdx.x * BS_THREADS + threadIdx.x; v < nvec; v += stride) {
    const uint4 wi = reinterpret_cast<const uint4*>(in)[v];
    const uint4 wo = reinterpret_cast<const uint4*>(out)[v];
    const uint2 pq = has_prev ? reinterpret_cast<const uint2*>(dprev_q)[v] : make_uint2(0u, 0u);
    const int ep = has_prev ? (int)dprev_s[v >> 2] - 127 : 0;
    uint32_t codes[2];
    int e;
    mx8_vector(a, wi, wo, has_prev, pq, ep, codes, e);
    if (dnew_q) {
      reinterpret_cast<uint2*>(dnew_q)[v] = make_uint2(codes[0], codes[1]);
      if ((threadIdx.x & 3) == 0) dnew_s[v >> 2] = (uint8_t)(e + 127);
    }
  }
  bs_finish<BS_GRID_MX8>(a, part, counter, stats);
}

size_t bs_workspace_bytes(int64_t n) {
  (void)n;
  return BS_HEADER + (size_t)std::max(BS_GRID_BF16, BS_GRID_MX8) * 8 * sizeof(double);
}

hipError_t launch_block_stats(const void* in, const void* out, const void* dprev, void* dnew,
                              int64_t n, double* stats, void* ws, hipStream_t st) {
  const int grid = bs_grid(n);
  unsigned* counter = static_cast<unsigned*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + BS_HEADER);
  if (dprev)
    hipLaunchKernelGGL(block_stats_kernel<true>, dim3(grid), dim3(BS_THREADS), 0, st,
                       static_cast<const uint16_t*>(in), static_cast<const uint16_t*>(out),
                       static_cast<const uint16_t*>(dprev), static_cast<uint16_t*>(dnew), n, part, counter, stats);
  else
    hipLaunchKernelGGL(block_stats_kernel<false>, dim3(grid), dim3(BS_THREADS), 0, st,
                       static_cast<const uint16_t*>(in), static_cast<const uint16_t*>(out), nullptr,
                       static_cast<uint16_t*>(dnew), n, part, counter, stats);
  return hipGetLastError();
}

hipError_t launch_block_stats_mx8(const void* in, const void* out, const uint8_t* dprev_q, const uint8_t* dprev_s,
                                  uint8_t* dnew_q, uint8_t* dnew_s, int64_t n, double* stats, void* ws,
                                  hipStream_t st) {
  // whole workgroups of 256 lanes: a multiple of 4 lanes per block
  const int grid = bs_grid_mx8(n);
  unsigned* counter = static_cast<unsigned*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + BS_HEADER);
  hipLaunchKernelGGL(block_stats_mx8_kernel, dim3(grid), dim3(BS_THREADS), 0, st,
                     static_cast<const uint16_t*>(in), static_cast<const uint16_t*>(out), dprev_q, dprev_s,
                     dnew_q, dnew_s, n, part, counter, stats);
  return hipGetLastError();
}

}  // namespace vdtq
