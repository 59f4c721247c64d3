// Online block Hadamard transform + NVFP4 / per-token INT8 / MX (MXFP4,
// MXFP8) quantization of bf16 activations, with the outlier statistics fused
// in (gfx950).
//
// The operation: gist.science "6Bit-Diffusion: Inference-Time Mixed-Precision
// Quantization for Video Diffusion Models" §2.A (block Hadamard before
// quantization; NVFP4 for stable blocks, INT8 for volatile ones) and
// youleyou.com "清华大学6Bit-Diffusion技术..." §一 and §三 (max/mean outlier
// ratio of the input); fused into one pass as §4 / §四 describe.
//
// Design (HBM-bound pass, 2 B/element in, 0.5625 (NVFP4) or 1 (INT8) out):
//   * A 128-thread workgroup owns 128 "chunks" of 64 consecutive elements of
//     a row (small workgroups: 16 KB of LDS each, so registers set the
//     occupancy, and a short last wave).  The chunks are staged through LDS
//     with fully coalesced 16-byte loads (a wavefront reads 1 KB contiguous
//     per instruction) and an XOR swizzle, so that each thread then reads its
//     own 128-byte chunk without bank conflicts.
//   * Every thread keeps its 64 values in registers and runs the butterflies
//     h = 1, 2, ..., min(b, 64)/2 in fp32 with no data exchange; for b = 128
//     and 256 the remaining stages pair neighbouring lanes with one shuffle.
//   * A 16-element NVFP4 group lies inside a thread, so group maxima are
//     register-local.  Each group costs one correctly rounded division (the
//     E4M3 scale) and a table read (its reciprocal); each element costs one
//     multiply and half of a hardware E2M1 conversion
//     (v_cvt_scalef32_pk_fp4_f32, whose power-of-two scale operand also
//     absorbs the 1/sqrt(b) normalisation when b is a power of four).
//   * INT8: a workgroup owns whole rows (192 or 256 threads, whichever
//     leaves fewer lanes idle); the row maximum is combined with LDS atomic
//     max on the float bits (order independent), and rint is the
//     2^23-magic-number add whose low byte is the two's complement code.
//   * MX (OCP Microscaling v1.0 conversion; the variant of NVFP4 / INT8 for
//     block-scaled matrix instructions): a thread's chunk is two 32-element
//     blocks; the E8M0 exponent comes from the block maximum's exponent
//     field, elements are scaled by exact powers of two and converted by the
//     hardware (E2M1 saturates by itself; E4M3 is clamped to +-448 first,
//     the conversion itself does not saturate).  No tensor scale, one pass.
//   * GELU prologue (flag 4; the FFN-down input taken straight from FFN-up's
//     bf16 output): each element is replaced by the bf16 GELU of
//     hadamard_common.h before anything else: a table of subtrahends
//     (written once per call, copied into LDS) indexed two elements at a
//     time with packed 16-bit arithmetic.
//   * Statistics: fp32 over a thread's 64 elements, fp64 across threads and
//     workgroups in a fixed order (bit-reproducible, no float atomics).
#include <algorithm>
#include <mutex>

#include "../../include/vdtq.h"

#include "device_common.h"
#include "hadamard_common.h"
#include "launch.h"

namespace vdtq {

constexpr int HQ_THREADS = 128;

struct HQParams {
  const uint16_t* x;
  int64_t ldx;
  int32_t M, K, cpr;          // cpr = chunks of 64 per row = ceil(K / 64)
  int32_t rows_per_wg;        // INT8: whole rows per workgroup
  int64_t total_chunks;       // M * cpr
  double inv_cpr;             // 1 / cpr, for the quotient estimate
  uint8_t* q;
  void* scales;
  float* ts;                  // NVFP4 {amax_T, gs}
  float* amax_part;           // [grid] partial maxima (amax pre-pass)
  double* stats_part;         // [grid][4] partial statistics
  unsigned flags;
  int32_t flat;               // ldx == K and K % 64 == 0: chunk g starts at element 64 g
  const uint16_t* gtab;       // the device's GELU table (flag 4)
};

__device__ __forceinline__ void divmod_cpr(int64_t g, const HQParams& p, int& row, int& col) {
  int64_t r = (int64_t)((double)g * p.inv_cpr);
  int64_t c = g - r * p.cpr;
  if (c < 0) { --r; c += p.cpr; }
  if (c >= p.cpr) { ++r; c -= p.cpr; }
  row = (int)r;
  col = (int)c;
}

// ---------------------------------------------------------------- staging
// Loads the workgroup's T chunks (T = its thread count) into LDS (zeros
// where the chunk or the 8-element slot lies outside X) and returns this
// thread's own chunk coordinates.  ROWS: chunks are rows_per_wg whole rows;
// otherwise the workgroup owns flat chunk ids [T wg, T wg + T).  mid() runs
// after the global loads are issued and before their data is needed, so
// independent set-up work overlaps their latency.
struct NoMid {
  __device__ void operator()() const {}
};

template <bool ROWS, int T = HQ_THREADS, class Mid = NoMid>
__device__ __forceinline__ void stage(const HQParams& p, uint4* lds, int& my_row, int& my_col,
                                      bool& my_valid, int wg = blockIdx.x, Mid mid = Mid()) {
  const int t = threadIdx.x;
  const int j = t & 7;
  int row, col;
  int c0 = t >> 3;
  if (p.flat) {
    // contiguous whole-chunk rows: the workgroup's chunks are one contiguous
    // run starting at chunk g0, so loads need no row / column arithmetic
    const int chunk_limit = ROWS ? p.rows_per_wg * p.cpr : T;
    const int64_t g0 = ROWS ? (int64_t)wg * p.rows_per_wg * p.cpr : (int64_t)wg * T;
    const int64_t left = p.total_chunks - g0;
    const int lim = (int)min<int64_t>(chunk_limit, left);
    // The run is read through a buffer resource of lim chunks: the hardware
    // returns zeros past its end, so the eight loads need no branch and no
    // merge with a zero value (which made the compiler wait for the first
    // loads before issuing the rest).
    const __amdgpu_buffer_rsrc_t run = raw_buffer(p.x + g0 * 64, (uint32_t)lim * 128u);
    const uint32_t off = (uint32_t)(c0 * 128 + 16 * j);
    uint4 buf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) buf[i] = buffer_load16(run, off + i * ((T / 8) * 128));
    mid();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + (T / 8) * i;
      lds[c * 8 + (j ^ (c & 7))] = buf[i];
    }
    if (ROWS) {
      divmod_cpr(t, p, my_row, my_col);
      my_row += wg * p.rows_per_wg;
      my_valid = t < lim;
    } else {
      divmod_cpr(g0 + t, p, my_row, my_col);
      my_valid = t < lim;
    }
    return;
  }
  if (ROWS) {
    divmod_cpr(c0, p, row, col);
    row += wg * p.rows_per_wg;
  } else {
    divmod_cpr((int64_t)wg * T + c0, p, row, col);
  }
  const int chunk_limit = ROWS ? p.rows_per_wg * p.cpr : T;
  uint4 buf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c0 + (T / 8) * i;
    const int e = col * 64 + 8 * j;
    const bool ok = (c < chunk_limit) && (row < p.M) && (e < p.K);
    buf[i] = ok ? *reinterpret_cast<const uint4*>(p.x + (int64_t)row * p.ldx + e)
                : make_uint4(0u, 0u, 0u, 0u);
    col += T / 8;
    while (col >= p.cpr) { col -= p.cpr; ++row; }
  }
  mid();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c0 + (T / 8) * i;
    lds[c * 8 + (j ^ (c & 7))] = buf[i];
  }
  if (ROWS) {
    divmod_cpr(t, p, my_row, my_col);
    my_row += wg * p.rows_per_wg;
    my_valid = (t < chunk_limit) && (my_row < p.M);
  } else {
    divmod_cpr((int64_t)wg * T + t, p, my_row, my_col);
    my_valid = my_row < p.M;
  }
}

// With the GELU flag (4) each quantize workgroup copies the GELU table from
// the device's table (gelu_table below) into dynamic LDS (gelu_lds) while
// its chunk loads are in flight (the stage() hook); load_chunk maps each
// staged element through it as it widens the chunk.
extern __shared__ __attribute__((aligned(16))) uint16_t gelu_lds[];

__global__ __launch_bounds__(256) void gelu_table_kernel(uint16_t* tab) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < kGeluTabN) tab[i] = gelu_table_entry(i);
}

__device__ __forceinline__ void gelu_begin(const HQParams& p) {
  if (!(p.flags & 4u)) return;
  for (int i = threadIdx.x; i < kGeluTabBytes / 16; i += blockDim.x)
    reinterpret_cast<uint4*>(gelu_lds)[i] = reinterpret_cast<const uint4*>(p.gtab)[i];
}

// Reads this thread's chunk from LDS and widens bf16 -> fp32 (through the
// GELU table first with flag 4).
__device__ __forceinline__ void load_chunk(const uint4* lds, float (&v)[64], unsigned flags) {
  const int t = threadIdx.x;
  const bool gelu = (flags & 4u) != 0;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    uint4 w = lds[t * 8 + (jj ^ (t & 7))];
    if (gelu)
      w = make_uint4(gelu_word(w.x, gelu_lds), gelu_word(w.y, gelu_lds), gelu_word(w.z, gelu_lds),
                     gelu_word(w.w, gelu_lds));
    v[8 * jj + 0] = bf16_lo(w.x); v[8 * jj + 1] = bf16_hi(w.x);
    v[8 * jj + 2] = bf16_lo(w.y); v[8 * jj + 3] = bf16_hi(w.y);
    v[8 * jj + 4] = bf16_lo(w.z); v[8 * jj + 5] = bf16_hi(w.z);
    v[8 * jj + 6] = bf16_lo(w.w); v[8 * jj + 7] = bf16_hi(w.w);
  }
}

// Eight E2M1 codes of RN(v[i] * inv) / sc (sc a power of two, exact), packed
// low nibble first: the hardware conversion rounds to nearest even,
// saturates at 6 and keeps the sign of zero.
__device__ __forceinline__ uint32_t pack8_e2m1(const float* v, float inv, float sc) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * inv, v[1] * inv, sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * inv, v[3] * inv, sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * inv, v[5] * inv, sc, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * inv, v[7] * inv, sc, 3);
  return w;
}

// ---------------------------------------------------------------- statistics
__device__ __forceinline__ void input_stats(const float (&v)[64], int nvalid, float& mx, float& sx) {
  mx = 0.0f;
  sx = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float a = (i < nvalid) ? fabsf(v[i]) : 0.0f;
    mx = fmaxf(mx, a);
    sx = sx + a;
  }
}

// Sum / max of four per-thread values over the workgroup, fp64, fixed order;
// thread 0 writes them to part[4].
template <int T = HQ_THREADS>
__device__ void wg_stats_write(double mx, double sx, double my, double sy, double* part) {
  __shared__ double red[4][T / 64];
  mx = wave_max_d(mx);
  sx = wave_sum(sx);
  my = wave_max_d(my);
  sy = wave_sum(sy);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = mx; red[1][w] = sx; red[2][w] = my; red[3][w] = sy; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = red[0][0], b = red[1][0], c = red[2][0], d = red[3][0];
    for (int i = 1; i < T / 64; ++i) {
      a = fmax(a, red[0][i]); b += red[1][i]; c = fmax(c, red[2][i]); d += red[3][i];
    }
    part[0] = a; part[1] = b; part[2] = c; part[3] = d;
  }
}

// ---------------------------------------------------------------- amax pre-pass
// The workgroups walk the tensor from its end (workgroup i takes tile
// G - 1 - i): the quantize pass that follows starts at the front, which is
// then what the last-level cache holds.  The maximum does not depend on the
// order.  STATS: the pass also takes the outlier statistics (it transforms
// every value anyway), in the quantize pass's per-thread order (sums of 16
// |y| per group); staged zeros pad the tail and add nothing to any of them.
template <int B, bool STATS>
__global__ __launch_bounds__(HQ_THREADS) void hq_amax_kernel(HQParams p) {
  __shared__ uint4 lds[HQ_THREADS * 8];
  __shared__ float wred[HQ_THREADS / 64];
  int row, col;
  bool valid;
  stage<false>(p, lds, row, col, valid, (int)(gridDim.x - 1 - blockIdx.x), [&]() { gelu_begin(p); });
  __syncthreads();
  float v[64];
  load_chunk(lds, v, p.flags);
  float mx = 0.0f, sx = 0.0f;
  if (STATS) {
    input_stats(v, 64, mx, sx);
    // taken here, before the butterflies overwrite v (left to the scheduler,
    // the input values were kept in a second set of registers)
    asm volatile("" : "+v"(mx), "+v"(sx));
  }
  fwht<B>(v);
  normalise<B>(v);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(v[i]));   // staged zeros pad the tail
  float sy = 0.0f;
  if (STATS) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s = s + fabsf(v[16 * g + e]);
      sy = sy + s * yfac<B>();
    }
  }
  const float my = m * yfac<B>();                 // exact (power of two)
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = wred[0];
    for (int i = 1; i < HQ_THREADS / 64; ++i) a = fmaxf(a, wred[i]);
    p.amax_part[blockIdx.x] = a * yfac<B>();
  }
  if (STATS) wg_stats_write(mx, sx, my, sy, p.stats_part + 4 * (int64_t)blockIdx.x);
}

// One workgroup of kFinalThreads: amax_T = max of the partial maxima;
// writes {amax_T, gs}.  Each thread keeps 16 loads in flight; reads past n
// are zeros, neutral for a maximum of non-negative values.
constexpr int kFinalThreads = 1024;

__device__ __forceinline__ void amax_final(const float* part, int n, float* ts) {
  __shared__ float wred[kFinalThreads / 64];
  constexpr int U = 16;
  const __amdgpu_buffer_rsrc_t r = raw_buffer(part, (uint32_t)n * 4u);
  float m = 0.0f;
  for (int base = 0; base < n; base += U * kFinalThreads) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = buffer_load4f(r, (uint32_t)(base + u * kFinalThreads + threadIdx.x) * 4u);
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, x[u]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = wred[0];
    for (int w = 1; w < kFinalThreads / 64; ++w) a = fmaxf(a, wred[w]);
    ts[0] = a;
    ts[1] = nvfp4_gs(a);
  }
}

__global__ __launch_bounds__(kFinalThreads) void hq_amax_final_kernel(const float* part, int n, float* ts) {
  amax_final(part, n, ts);
}

// Writes gs for a caller-supplied amax (used when there are no rows).
__global__ void hq_gs_only_kernel(float* ts) {
  if (threadIdx.x == 0) ts[1] = nvfp4_gs(ts[0]);
}

// Final fp64 reduction of the per-workgroup statistics {max, sum, max, sum}
// (fixed order).  Each thread keeps 4 partials (8 loads) in flight; reads
// past n are zeros, neutral for these non-negative maxima and sums.
__device__ __forceinline__ void stats_final(const double* part, int n, double* out) {
  __shared__ double red[4][kFinalThreads / 64];
  constexpr int U = 4;
  const __amdgpu_buffer_rsrc_t r = raw_buffer(part, (uint32_t)n * 32u);
  double a = 0.0, b = 0.0, c = 0.0, d = 0.0;
  for (int base = 0; base < n; base += U * kFinalThreads) {
    uint4 w[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)(base + u * kFinalThreads + threadIdx.x) * 32u;
      w[u][0] = buffer_load16(r, off);
      w[u][1] = buffer_load16(r, off + 16u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a = fmax(a, u2d(w[u][0].x, w[u][0].y));
      b += u2d(w[u][0].z, w[u][0].w);
      c = fmax(c, u2d(w[u][1].x, w[u][1].y));
      d += u2d(w[u][1].z, w[u][1].w);
    }
  }
  a = wave_max_d(a); b = wave_sum(b); c = wave_max_d(c); d = wave_sum(d);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = a; red[1][w] = b; red[2][w] = c; red[3][w] = d; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double x0 = red[0][0], x1 = red[1][0], x2 = red[2][0], x3 = red[3][0];
    for (int i = 1; i < kFinalThreads / 64; ++i) {
      x0 = fmax(x0, red[0][i]); x1 += red[1][i]; x2 = fmax(x2, red[2][i]); x3 += red[3][i];
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
  }
}

__global__ __launch_bounds__(kFinalThreads) void hq_stats_final_kernel(const double* part, int n, double* out) {
  stats_final(part, n, out);
}

// Both reductions of an amax pre-pass that also took the statistics.
__global__ __launch_bounds__(kFinalThreads) void hq_amax_stats_final_kernel(const float* apart, const double* spart,
                                                                            int n, float* ts, double* out) {
  amax_final(apart, n, ts);
  stats_final(spart, n, out);
}

// NVFP4 encoding of a thread's 64 transformed register values: per 16-group
// the E4M3 scale byte (byte g of sbytes) and 16 E2M1 codes (words 2g, 2g+1);
// with want_stats, max|y| and sum|y| over the first nvalid values are folded
// into my / sy.
template <int B>
__device__ __forceinline__ void nvfp4_encode64(const float (&v)[64], const float* inv_tab, bool ok, float d,
                                               bool want_stats, int nvalid, uint32_t (&words)[8],
                                               uint32_t& sbytes, float& my, float& sy) {
  sbytes = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float av = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) av = fmaxf(av, fabsf(v[16 * g + e]));
    const float ag = av * yfac<B>();                 // exact (power of two)
    uint32_t s8 = ok ? e4m3_encode_pos(ag / d) : 0u;
    const float inv = inv_tab[s8];                  // 0 exactly when s_dec == 0
    const bool nz = inv != 0.0f;
    const uint32_t w0 = pack8_e2m1(&v[16 * g], inv, HadScale<B>::inv);
    const uint32_t w1 = pack8_e2m1(&v[16 * g + 8], inv, HadScale<B>::inv);
    words[2 * g] = nz ? w0 : 0u;
    words[2 * g + 1] = nz ? w1 : 0u;
    sbytes |= s8 << (8 * g);
    if (want_stats && 16 * g < nvalid) {
      my = fmaxf(my, ag);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s = s + fabsf(v[16 * g + e]);
      sy = sy + s * yfac<B>();
    }
  }
}

// ---------------------------------------------------------------- NVFP4 pass
// STATS: the fused statistics (flag 2) are compiled in only where asked for,
// so the plain pass fits four waves per SIMD.
template <int B, bool STATS>
__global__ __launch_bounds__(HQ_THREADS) void hq_nvfp4_kernel(HQParams p) {
  __shared__ uint4 lds[HQ_THREADS * 8];
  __shared__ float inv_tab[128];
  float amax = 0.0f, gs = 1.0f;
  bool ok = false;
  // under the chunk loads: the tensor scale, and RN(1 / s_dec) for every
  // E4M3 code (s_dec = RN(e4m3 * gs), 0 -> 0), so that the per-group
  // reciprocal is a table read (one entry per thread)
  static_assert(HQ_THREADS == 128, "one reciprocal-table entry per thread");
  auto scale_setup = [&]() {
    amax = p.ts[0];
    ok = nvfp4_amax_ok(amax);
    gs = ok ? amax / 2688.0f : 1.0f;
    const float sd = e4m3_decode_pos(threadIdx.x) * gs;
    inv_tab[threadIdx.x] = sd != 0.0f ? 1.0f / sd : 0.0f;
  };
  int row, col;
  bool valid;
  stage<false>(p, lds, row, col, valid, blockIdx.x, [&]() {
    gelu_begin(p);
    scale_setup();
  });
  __syncthreads();
  float v[64];
  load_chunk(lds, v, p.flags);
  const int nvalid = valid ? min(64, p.K - col * 64) : 0;
  const bool want_stats = STATS && (p.flags & 2u) != 0;
  float mx = 0.0f, sx = 0.0f;
  if (want_stats) input_stats(v, nvalid, mx, sx);
  fwht<B>(v);
  normalise<B>(v);

  const float d = 6.0f * gs;
  if (blockIdx.x == 0 && threadIdx.x == 0) p.ts[1] = gs;

  uint32_t words[8];
  uint32_t sbytes;
  float my = 0.0f, sy = 0.0f;
  nvfp4_encode64<B>(v, inv_tab, ok, d, want_stats, nvalid, words, sbytes, my, sy);

  if (valid && p.flat) {
    // contiguous whole chunks: chunk g's codes at 32 g, its scales at 4 g
    // (a workgroup-uniform base plus a 32-bit lane offset)
    const int64_t wg0 = (int64_t)blockIdx.x * HQ_THREADS;
    reinterpret_cast<uint4*>(p.q + wg0 * 32)[2 * threadIdx.x] = make_uint4(words[0], words[1], words[2], words[3]);
    reinterpret_cast<uint4*>(p.q + wg0 * 32)[2 * threadIdx.x + 1] = make_uint4(words[4], words[5], words[6], words[7]);
    reinterpret_cast<uint32_t*>(p.scales)[wg0 + threadIdx.x] = sbytes;
  } else if (valid) {
    uint8_t* qrow = p.q + (int64_t)row * (p.K / 2) + col * 32;
    uint8_t* srow = reinterpret_cast<uint8_t*>(p.scales) + (int64_t)row * (p.K / 16) + col * 4;
    if (nvalid == 64 && (p.K % 32) == 0) {
      reinterpret_cast<uint4*>(qrow)[0] = make_uint4(words[0], words[1], words[2], words[3]);
      reinterpret_cast<uint4*>(qrow)[1] = make_uint4(words[4], words[5], words[6], words[7]);
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (16 * g < nvalid) reinterpret_cast<uint2*>(qrow)[g] = make_uint2(words[2 * g], words[2 * g + 1]);
    }
    if (nvalid == 64 && (p.K % 64) == 0) {
      *reinterpret_cast<uint32_t*>(srow) = sbytes;
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (16 * g < nvalid) srow[g] = (uint8_t)(sbytes >> (8 * g));
    }
  }
  if (want_stats) wg_stats_write(mx, sx, my, sy, p.stats_part + 4 * (int64_t)blockIdx.x);
}

// ---------------------------------------------------------------- INT8 pass
// T threads per workgroup, rows_per_wg * cpr <= T chunks (the launcher picks
// T = 192 or 256, whichever leaves fewer lanes idle).
template <int B, int T>
__global__ __launch_bounds__(T) void hq_int8_kernel(HQParams p) {
  __shared__ uint4 lds[T * 8];
  __shared__ uint32_t rowmax[T];
  int row, col;
  bool valid;
  // the row maxima are cleared while the chunk loads are in flight; the
  // barrier after staging orders the clear before the atomics
  stage<true, T>(p, lds, row, col, valid, blockIdx.x, [&]() {
    gelu_begin(p);
    if (threadIdx.x < p.rows_per_wg) rowmax[threadIdx.x] = 0u;
  });
  __syncthreads();
  float v[64];
  load_chunk(lds, v, p.flags);
  const int nvalid = valid ? min(64, p.K - col * 64) : 0;
  const bool want_stats = (p.flags & 2u) != 0;
  float mx = 0.0f, sx = 0.0f;
  if (want_stats) input_stats(v, nvalid, mx, sx);
  fwht<B>(v);
  normalise<B>(v);

  float av = 0.0f, sv = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) av = fmaxf(av, fabsf(v[i]));   // padded slots are 0
  const float ay = av * yfac<B>();
  const int rl = row - blockIdx.x * p.rows_per_wg;
  if (valid) atomicMax(&rowmax[rl], __float_as_uint(ay));
  __syncthreads();
  const float a = valid ? __uint_as_float(rowmax[rl]) : 0.0f;
  const bool ok = (a == a) && a >= kZeroLimit && a <= 3.0e38f;
  const float s = ok ? a / 127.0f : 0.0f;
  const float inv = ok ? 1.0f / s : 0.0f;
  // rint_even(y * inv) with y = v * 2^-k: RN(v * inv) + 1.5 * 2^(23 + k) rounds
  // at unit 2^k, and the low byte of the sum's bits is the int8 code.
  constexpr float magic = 12582912.0f * HadScale<B>::inv;
  uint32_t words[16];
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    uint32_t b0 = __float_as_uint(v[4 * w + 0] * inv + magic);
    uint32_t b1 = __float_as_uint(v[4 * w + 1] * inv + magic);
    uint32_t b2 = __float_as_uint(v[4 * w + 2] * inv + magic);
    uint32_t b3 = __float_as_uint(v[4 * w + 3] * inv + magic);
    uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    words[w] = ok ? (lo | (hi << 16)) : 0u;
  }
  if (p.flat) {
    // The workgroup's codes are one contiguous run of its chunks (64 bytes
    // each).  They leave through LDS so that every store instruction writes
    // consecutive 16-byte vectors, not 16 bytes every 64.  The staging buffer
    // is free: every thread read its chunk before the row-maximum barrier.
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds[4 * t + (i ^ (t & 3))] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    __syncthreads();
    const int64_t g0 = (int64_t)blockIdx.x * p.rows_per_wg * p.cpr;
    const int lim = (int)min<int64_t>((int64_t)p.rows_per_wg * p.cpr, p.total_chunks - g0);
    uint4* dst = reinterpret_cast<uint4*>(p.q + g0 * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v16 = t + T * i;                       // 16-byte vector of the run
      const int c = v16 >> 2, jj = v16 & 3;
      if (v16 < 4 * lim) dst[v16] = lds[4 * c + (jj ^ (c & 3))];
    }
    if (valid && col == 0) reinterpret_cast<float*>(p.scales)[row] = s;
  } else if (valid) {
    int8_t* qrow = reinterpret_cast<int8_t*>(p.q) + (int64_t)row * p.K + col * 64;
    for (int g = 0; g < 4; ++g)
      if (16 * g < nvalid)
        reinterpret_cast<uint4*>(qrow)[g] =
            make_uint4(words[4 * g], words[4 * g + 1], words[4 * g + 2], words[4 * g + 3]);
    if (col == 0) reinterpret_cast<float*>(p.scales)[row] = s;
  }
  if (want_stats) {
    float my = valid ? ay : 0.0f;
    for (int i = 0; i < 64; ++i) sv = sv + ((i < nvalid) ? fabsf(v[i]) : 0.0f);
    wg_stats_write<T>(mx, sx, my, (double)(sv * yfac<B>()), p.stats_part + 4 * (int64_t)blockIdx.x);
  }
}

// ---------------------------------------------------------------- BF16 pass
// The full-precision fallback: the rotated activations rounded to bf16
// (nearest even), flat chunks as in the NVFP4 pass.
template <int B>
__global__ __launch_bounds__(HQ_THREADS) void hq_bf16_kernel(HQParams p) {
  __shared__ uint4 lds[HQ_THREADS * 8];
  int row, col;
  bool valid;
  stage<false>(p, lds, row, col, valid, blockIdx.x, [&]() { gelu_begin(p); });
  __syncthreads();
  float v[64];
  load_chunk(lds, v, p.flags);
  const int nvalid = valid ? min(64, p.K - col * 64) : 0;
  const bool want_stats = (p.flags & 2u) != 0;
  float mx = 0.0f, sx = 0.0f;
  if (want_stats) input_stats(v, nvalid, mx, sx);
  fwht<B>(v);
  normalise<B>(v);
  constexpr float f = yfac<B>();                     // exact power of two (1 when applied)
  uint32_t words[32];
#pragma unroll
  for (int w = 0; w < 32; ++w)
    words[w] = f32_to_bf16_bits(v[2 * w] * f) | (f32_to_bf16_bits(v[2 * w + 1] * f) << 16);
  if (valid) {
    uint4* qrow = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.q) + (int64_t)row * p.K + col * 64);
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (8 * g < nvalid)
        qrow[g] = make_uint4(words[4 * g], words[4 * g + 1], words[4 * g + 2], words[4 * g + 3]);
  }
  if (want_stats) {
    float my = 0.0f, sy = 0.0f;
    for (int i = 0; i < 64; ++i) {
      const float a = (i < nvalid) ? fabsf(v[i]) : 0.0f;
      my = fmaxf(my, a);
      sy = sy + a;
    }
    wg_stats_write(mx, sx, (double)(my * f), (double)(sy * f), p.stats_part + 4 * (int64_t)blockIdx.x);
  }
}

// ---------------------------------------------------------------- MX pass
template <int B, bool FP8>
__global__ __launch_bounds__(HQ_THREADS) void hq_mx_kernel(HQParams p) {
  __shared__ uint4 lds[HQ_THREADS * 8];
  int row, col;
  bool valid;
  stage<false>(p, lds, row, col, valid, blockIdx.x, [&]() { gelu_begin(p); });
  __syncthreads();
  float v[64];
  load_chunk(lds, v, p.flags);
  const int nvalid = valid ? min(64, p.K - col * 64) : 0;
  const bool want_stats = (p.flags & 2u) != 0;
  float mx = 0.0f, sx = 0.0f;
  if (want_stats) input_stats(v, nvalid, mx, sx);
  fwht<B>(v);
  normalise<B>(v);
  uint32_t words[FP8 ? 16 : 8];
  uint32_t sbytes;
  mx_encode64<B, FP8>(v, words, sbytes);

  if (FP8 && p.flat) {
    // E4M3 codes, 64 bytes per chunk: the workgroup's run leaves through LDS
    // so that every store instruction writes consecutive 16-byte vectors
    const int t = threadIdx.x;
    __syncthreads();                                     // every chunk has been read from lds
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds[4 * t + (i ^ (t & 3))] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    __syncthreads();
    const int64_t g0 = (int64_t)blockIdx.x * HQ_THREADS;
    const int lim = (int)min<int64_t>(HQ_THREADS, p.total_chunks - g0);
    uint4* dst = reinterpret_cast<uint4*>(p.q + g0 * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v16 = t + HQ_THREADS * i;
      const int c = v16 >> 2, jj = v16 & 3;
      if (v16 < 4 * lim) dst[v16] = lds[4 * c + (jj ^ (c & 3))];
    }
    if (valid) *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(p.scales) + (g0 + t) * 2) = (uint16_t)sbytes;
  } else if (valid) {
    constexpr int BYTES = FP8 ? 64 : 32;                      // code bytes per chunk
    uint4* qrow = reinterpret_cast<uint4*>(p.q + (int64_t)row * (FP8 ? p.K : p.K / 2) + col * BYTES);
    uint8_t* srow = reinterpret_cast<uint8_t*>(p.scales) + (int64_t)row * (p.K / 32) + col * 2;
    const int nq = (nvalid == 64 ? BYTES : BYTES / 2) / 16;  // a 32-element tail chunk: first block only
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i)
      if (i < nq) qrow[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    if (nvalid == 64 && (p.K % 64) == 0)
      *reinterpret_cast<uint16_t*>(srow) = (uint16_t)sbytes;
    else
      for (int b = 0; 32 * b < nvalid; ++b) srow[b] = (uint8_t)(sbytes >> (8 * b));
  }
  if (want_stats) {
    constexpr float f = yfac<B>();
    float my = 0.0f, sy = 0.0f;
    for (int i = 0; i < 64; ++i) {
      const float a = (i < nvalid) ? fabsf(v[i]) : 0.0f;
      my = fmaxf(my, a);
      sy = sy + a;
    }
    wg_stats_write(mx, sx, (double)(my * f), (double)(sy * f), p.stats_part + 4 * (int64_t)blockIdx.x);
  }
}

// ---------------------------------------------------------------- launcher
// INT8 workgroup size for rows of cpr chunks (cpr <= 256): 192 threads when
// floor(192 / cpr) whole rows leave fewer lanes idle than floor(256 / cpr)
// rows in 256 threads, else 256 (64 or 128 threads never do better than 256,
// which holds twice or four times their rows).
static int hq_int8_threads(int cpr) {
  const int r192 = 192 / cpr, r256 = 256 / cpr;
  return (r192 >= 1 && r192 * cpr * 256 > r256 * cpr * 192) ? 192 : 256;
}

// stats: where the statistics' final reduction goes (the partials are
// written by this call's kernels).  NVFP4 with the tensor amax computed takes
// them in the pre-pass and reduces both in one launch; otherwise the pass
// takes them and the final kernel follows it.
template <int B>
static hipError_t launch_b(const HQParams& p, int fmt, bool amax_given, int grid, double* stats, hipStream_t st) {
  const size_t shm = (p.flags & 4u) ? (size_t)kGeluTabBytes : 0;   // the GELU table
  const bool want_stats = (p.flags & 2u) != 0;
  if (fmt == 0 && !amax_given) {
    if (want_stats) {
      hipLaunchKernelGGL((hq_amax_kernel<B, true>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
      hipLaunchKernelGGL(hq_amax_stats_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, p.amax_part, p.stats_part,
                         grid, p.ts, stats);
    } else {
      hipLaunchKernelGGL((hq_amax_kernel<B, false>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
      hipLaunchKernelGGL(hq_amax_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, p.amax_part, grid, p.ts);
    }
    hipLaunchKernelGGL((hq_nvfp4_kernel<B, false>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
    return hipGetLastError();
  }
  if (fmt == 0) {
    if (want_stats)
      hipLaunchKernelGGL((hq_nvfp4_kernel<B, true>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
    else
      hipLaunchKernelGGL((hq_nvfp4_kernel<B, false>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
  } else if (fmt == 1) {
    if (hq_int8_threads(p.cpr) == 192)
      hipLaunchKernelGGL((hq_int8_kernel<B, 192>), dim3(grid), dim3(192), shm, st, p);
    else
      hipLaunchKernelGGL((hq_int8_kernel<B, 256>), dim3(grid), dim3(256), shm, st, p);
  } else if (fmt == 2) {
    hipLaunchKernelGGL(hq_bf16_kernel<B>, dim3(grid), dim3(HQ_THREADS), shm, st, p);
  } else if (fmt == 3) {
    hipLaunchKernelGGL((hq_mx_kernel<B, false>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
  } else {
    hipLaunchKernelGGL((hq_mx_kernel<B, true>), dim3(grid), dim3(HQ_THREADS), shm, st, p);
  }
  if (want_stats) hipLaunchKernelGGL(hq_stats_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, p.stats_part, grid, stats);
  return hipGetLastError();
}

// Workspace: per-workgroup amax partials (float), then statistics partials
// (double[4]).
static size_t hq_partials_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 256;
  const int64_t cpr = (K + 63) / 64;
  // the largest grid of either format: flat chunks, or one row per group
  const int64_t grid = std::max<int64_t>((M * cpr + HQ_THREADS - 1) / HQ_THREADS, M);
  return (size_t)(((grid * 4 + 63) / 64) * 64 + grid * 4 * 8);
}

size_t hq_workspace_bytes(int64_t M, int64_t K) { return hq_partials_bytes(M, K); }

// ------------------------------------------------------------ GELU table
// One table per GPU, in the code object: it depends on nothing but the GELU
// definition, so it is built once per device and process, on the stream of
// the first call that needs it, which waits for the build (afterwards every
// kernel on any stream only reads it).  A call on a capturing stream may not
// wait: it records the build into the graph (every replay rebuilds the same
// values before using them) and leaves the table marked unbuilt.
static __device__ __align__(16) uint16_t gelu_tab_dev[kGeluTabBytes / 2];

hipError_t gelu_table(hipStream_t st, const uint16_t** tab) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  static bool built[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(gelu_tab_dev));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *tab = static_cast<const uint16_t*>(addr[dev]);
  if (built[dev]) return hipSuccess;
  hipLaunchKernelGGL(gelu_table_kernel, dim3((kGeluTabN + 255) / 256), dim3(256), 0, st,
                     static_cast<uint16_t*>(addr[dev]));
  e = hipGetLastError();
  if (e != hipSuccess || cs != hipStreamCaptureStatusNone) return e;
  e = hipStreamSynchronize(st);
  if (e == hipSuccess) built[dev] = true;
  return e;
}

// ------------------------------------------------ allocation-free scratch
// The workspace of hadamard_quantize_noalloc: a device array per GPU, in the
// code object (no allocation call), holding the partials exactly as a
// caller-given workspace would.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): it
// uses the device address hipGetSymbolAddress returns for the current
// device, looked up on the first call on each device and kept.
static __device__ __align__(256) uint8_t scratch[VDTQ_NOALLOC_SCRATCH_BYTES];

hipError_t hq_noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_hadamard_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, int b, int fmt,
                                    unsigned flags, void* q, void* scales, float* ts,
                                    double* stats, void* ws, hipStream_t st) {
  HQParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.cpr = (int32_t)((K + 63) / 64);
  p.inv_cpr = 1.0 / (double)p.cpr;
  p.total_chunks = M * p.cpr;
  p.q = static_cast<uint8_t*>(q);
  p.scales = scales;
  p.ts = ts;
  p.flags = flags;
  p.flat = (ldx == K) && (K % 64) == 0;
  const bool amax_given = (flags & 1u) != 0;
  const bool want_stats = (flags & 2u) != 0;
  int grid;
  if (fmt != 1) {
    grid = (int)((p.total_chunks + HQ_THREADS - 1) / HQ_THREADS);
  } else {
    p.rows_per_wg = std::max(1, hq_int8_threads(p.cpr) / p.cpr);
    grid = (int)((M + p.rows_per_wg - 1) / p.rows_per_wg);
  }
  char* wsb = static_cast<char*>(ws);
  const int64_t grid_cap = std::max<int64_t>((M * p.cpr + HQ_THREADS - 1) / HQ_THREADS, M);
  p.amax_part = reinterpret_cast<float*>(wsb);
  p.stats_part = reinterpret_cast<double*>(wsb + ((grid_cap * 4 + 63) / 64) * 64);

  if (M == 0) {
    if (fmt == 0) {
      if (amax_given)
        hipLaunchKernelGGL(hq_gs_only_kernel, dim3(1), dim3(64), 0, st, ts);
      else
        hipLaunchKernelGGL(hq_amax_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, p.amax_part, 0, ts);
    }
    if (want_stats) hipLaunchKernelGGL(hq_stats_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, p.stats_part, 0, stats);
    return hipGetLastError();
  }
  if (flags & 4u) {
    const hipError_t et = gelu_table(st, &p.gtab);
    if (et != hipSuccess) return et;
  }
  switch (b) {
    case 16: return launch_b<16>(p, fmt, amax_given, grid, stats, st);
    case 32: return launch_b<32>(p, fmt, amax_given, grid, stats, st);
    case 64: return launch_b<64>(p, fmt, amax_given, grid, stats, st);
    case 128: return launch_b<128>(p, fmt, amax_given, grid, stats, st);
    default: return launch_b<256>(p, fmt, amax_given, grid, stats, st);
  }
}

}  // namespace vdtq
