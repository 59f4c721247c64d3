// Host-side per-block scheduler of 6Bit-Diffusion: dynamic precision (DMPQ),
// temporal delta cache skips with an error accumulator (TDC), purified delta
// refresh (PDR) and the INT8 restart rule.
//
// gist.science "6Bit-Diffusion: Inference-Time Mixed-Precision Quantization
// for Video Diffusion Models": §2.A (low Gamma_{t-1} -> NVFP4, high -> INT8),
// §2.B (skip when Delta_{t-1} and Delta_{t-2} are similar; error-guided
// switching refreshes the cache), §2.C (outliers or temporal uncertainty force
// FP16/BF16 before a cache write).  youleyou.com article §三: outlier ratio =
// max / mean of the input; the first recompute after a skip runs INT8.
//
// Pure, deterministic host code: O(1) per block and step.
#include <math.h>

#include "../../include/vdtq.h"

extern "C" {

void dmpq_state_init(vdtq_dmpq_state* s) {
  if (!s) return;
  s->step = 0;
  s->has_d1 = s->has_d2 = s->skipped_last = s->has_gamma = 0;
  s->gamma_prev = 0.0;
  s->r_last = INFINITY;
  s->acc = 0.0;
}

double vdtq_outlier_ratio(double max_abs, double sum_abs, int64_t n) {
  if (sum_abs == 0.0 || n <= 0) return 1.0;
  return max_abs / (sum_abs / (double)n);
}

int dmpq_step(const vdtq_dmpq_params* p, vdtq_dmpq_state* s, const double* last_stats, double in_ratio,
              int* action) {
  if (!p || !s || !action) return VDTQ_EINVAL;
  if (last_stats) {
    // Gamma = ||out - in|| / ||in||; r = ||Dnew - Dprev|| / ||Dprev||
    const double d2 = last_stats[0], i2 = last_stats[1], dd2 = last_stats[2], p2 = last_stats[3];
    s->gamma_prev = (i2 == 0.0) ? (d2 == 0.0 ? 0.0 : INFINITY) : sqrt(d2 / i2);
    s->has_gamma = 1;
    if (s->has_d1) s->r_last = (p2 == 0.0) ? INFINITY : sqrt(dd2 / p2);
    s->has_d2 = s->has_d1;
    s->has_d1 = 1;
    s->skipped_last = 0;
    s->acc = 0.0;
  }
  const int64_t t = s->step++;
  if (t >= p->warmup && s->has_d2 && s->r_last < p->tau && s->acc + s->r_last < p->tau_acc) {
    s->acc += s->r_last;
    s->skipped_last = 1;
    *action = VDTQ_ACT_SKIP;
    return VDTQ_OK;
  }
  if (in_ratio > p->rho || (s->has_d2 && s->r_last > p->tau_u))
    *action = VDTQ_ACT_BF16;
  else if (s->skipped_last || !s->has_gamma || s->gamma_prev >= p->gamma)
    *action = VDTQ_ACT_INT8;
  else
    *action = VDTQ_ACT_NVFP4;
  return VDTQ_OK;
}

double dmpq_budget_gamma(const double* gammas, int32_t n, double avg_bits) {
  if (!gammas || n <= 0 || !isfinite(avg_bits)) return INFINITY;
  double kf = floor((double)n * (avg_bits - 4.0) / 4.0);
  if (kf <= 0.0) return INFINITY;
  const int32_t k = kf >= (double)n ? n : (int32_t)kf;
  // the k-th largest value: more than k-1 values are >= it and at most k-1
  // are strictly greater (O(n^2), n = blocks of a model; no allocation)
  for (int32_t i = 0; i < n; ++i) {
    int32_t greater = 0, at_least = 0;
    for (int32_t j = 0; j < n; ++j) {
      greater += gammas[j] > gammas[i];
      at_least += gammas[j] >= gammas[i];
    }
    if (greater < k && k <= at_least) return gammas[i];
  }
  return INFINITY;   // unreachable for comparable values
}

// Depth-aware caching profile (youleyou.com article §五: temporal stability
// differs with block depth): the skip thresholds scale linearly with the
// block's relative depth.
int dmpq_depth_params(const vdtq_dmpq_params* base, int32_t depth, int32_t n_blocks, double s_shallow,
                      double s_deep, vdtq_dmpq_params* out) {
  if (!base || !out || n_blocks <= 0 || depth < 0 || depth >= n_blocks) return VDTQ_EINVAL;
  if (!isfinite(s_shallow) || !isfinite(s_deep) || s_shallow < 0.0 || s_deep < 0.0) return VDTQ_EINVAL;
  const double d = n_blocks == 1 ? 0.0 : (double)depth / (double)(n_blocks - 1);
  const double s = s_shallow + (s_deep - s_shallow) * d;
  vdtq_dmpq_params r = *base;
  r.tau = base->tau * s;
  r.tau_acc = base->tau_acc * s;
  *out = r;
  return VDTQ_OK;
}

}  // extern "C"
