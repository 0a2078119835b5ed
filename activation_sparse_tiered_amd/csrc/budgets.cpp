// Host-side sparsity budgets: per-block targets from measured sensitivity (TopK-Guided,
// arXiv:2610.01763, section 2.2) and the greedy split of a block target over the block's
// projection groups (Appendix D, Table 4).  They produce the per-phase TopK-Guided targets
// the decode step's masks use; nothing here touches the GPU.
//
// Block targets: u_b = s + lambda (mean(sigma) - sigma_b) / mean(sigma); s_b = clamp(u_b + c,
// lo, hi) with the one shift c that keeps the mean of the targets at s, found by bisection
// (the mean is continuous and non-decreasing in c).  Greedy walk: increments
// alpha * mean(f) / f_m, so every increment moves the compute-weighted sparsity by
// alpha / n_mats; each round keeps the trial increment with the least block error (ties: the
// lower index), no matrix past sparsity 1, until P reaches P_max.
#include <cmath>
#include <vector>

#include "common.h"

using namespace spax;

namespace {

double compute_weighted(const double* f, const double* p, int n) {
  double num = 0.0, den = 0.0;
  for (int m = 0; m < n; ++m) {
    num += f[m] * p[m];
    den += f[m];
  }
  return num / den;
}

int block_sparsity_impl(const double* sens, int32_t n_blocks, double s, double lambda,
                        double s_min, double s_max, double* s_block) {
  if (!sens || !s_block) return fail(SPAX_ERR_NULL, "sens and s_block are required");
  if (n_blocks < 1) return fail(SPAX_ERR_PARAM, "n_blocks %d < 1", n_blocks);
  if (!std::isfinite(s) || !std::isfinite(lambda) || !std::isfinite(s_min) ||
      !std::isfinite(s_max) || lambda < 0 || s_min > s_max || s < s_min || s > s_max)
    return fail(SPAX_ERR_PARAM, "need 0 <= lambda and s_min <= s = %g <= s_max", s);
  double mean = 0.0;
  for (int b = 0; b < n_blocks; ++b) {
    if (!(sens[b] > 0) || !std::isfinite(sens[b]))
      return fail(SPAX_ERR_PARAM, "sensitivity %d is not finite and positive", b);
    mean += sens[b];
  }
  mean /= n_blocks;
  std::vector<double> u(n_blocks);
  double umin = INFINITY, umax = -INFINITY;
  for (int b = 0; b < n_blocks; ++b) {
    u[b] = s + lambda * (mean - sens[b]) / mean;
    umin = std::fmin(umin, u[b]);
    umax = std::fmax(umax, u[b]);
  }
  auto clamp = [&](double v) { return std::fmin(std::fmax(v, s_min), s_max); };
  auto mean_at = [&](double c) {
    double t = 0.0;
    for (int b = 0; b < n_blocks; ++b) t += clamp(u[b] + c);
    return t / n_blocks;
  };
  double a = s_min - umax - 1.0, z = s_max - umin + 1.0;
  for (int it = 0; it < 200; ++it) {
    const double m = 0.5 * (a + z);
    if (mean_at(m) < s) a = m;
    else z = m;
  }
  const double c = 0.5 * (a + z);
  for (int b = 0; b < n_blocks; ++b) s_block[b] = clamp(u[b] + c);
  return SPAX_OK;
}

int greedy_allocation_impl(const double* params, int32_t n_mats, double alpha, double P_max,
                           spax_block_error_fn block_error, void* user, double* rows,
                           int32_t cap, int32_t* n_rows) {
  if (!params || !block_error || !n_rows) return fail(SPAX_ERR_NULL, "params, block_error and n_rows are required");
  if (n_mats < 1 || n_mats > 64) return fail(SPAX_ERR_PARAM, "n_mats %d outside 1..64", n_mats);
  if (!(alpha > 0) || !std::isfinite(alpha) || !std::isfinite(P_max) || P_max > 1.0)
    return fail(SPAX_ERR_PARAM, "need alpha > 0 and P_max <= 1");
  if (cap < 0 || (cap > 0 && !rows)) return fail(SPAX_ERR_NULL, "rows is required when cap > 0");
  double fsum = 0.0;
  for (int m = 0; m < n_mats; ++m) {
    if (!(params[m] > 0) || !std::isfinite(params[m]))
      return fail(SPAX_ERR_PARAM, "parameter count %d is not finite and positive", m);
    fsum += params[m];
  }
  const double fmean = fsum / n_mats;
  std::vector<double> step(n_mats), p(n_mats, 0.0), trial(n_mats);
  double walk = 0.0;  // increments until every matrix is at sparsity 1
  for (int m = 0; m < n_mats; ++m) {
    step[m] = alpha * fmean / params[m];
    walk += 1.0 / step[m];
  }
  if (walk > 1e7) return fail(SPAX_ERR_PARAM, "alpha %g is too small: the walk could take %.3g "
                              "increments (limit 1e7)", alpha, walk);
  int32_t count = 0;
  auto record = [&]() {
    if (count < cap) {
      double* r = rows + (size_t)count * (1 + n_mats);
      r[0] = compute_weighted(params, p.data(), n_mats);
      for (int m = 0; m < n_mats; ++m) r[1 + m] = p[m];
    }
    ++count;
  };
  record();
  while (compute_weighted(params, p.data(), n_mats) < P_max) {
    int best = -1;
    double best_err = 0.0;
    for (int m = 0; m < n_mats; ++m) {
      if (p[m] + step[m] > 1.0 + 1e-12) continue;
      trial = p;
      trial[m] += step[m];
      const double e = block_error(trial.data(), n_mats, user);
      if (!std::isfinite(e)) {
        *n_rows = count;
        return fail(SPAX_ERR_PARAM, "block_error returned %g for a trial of matrix %d", e, m);
      }
      if (best < 0 || e < best_err) {
        best = m;
        best_err = e;
      }
    }
    if (best < 0) break;
    p[best] += step[best];
    record();
  }
  *n_rows = count;
  if (count > cap)
    return fail(SPAX_ERR_WORKSPACE, "the walk recorded %d rows; rows holds %d", count, cap);
  return SPAX_OK;
}
}  // namespace

extern "C" {

int spax_block_sparsity(const double* sens, int32_t n_blocks, double s, double lambda,
                        double s_min, double s_max, double* s_block) {
  clear_error();
  return no_throw(
      [&] { return block_sparsity_impl(sens, n_blocks, s, lambda, s_min, s_max, s_block); });
}

int spax_greedy_allocation(const double* params, int32_t n_mats, double alpha, double P_max,
                           spax_block_error_fn block_error, void* user, double* rows,
                           int32_t cap, int32_t* n_rows) {
  clear_error();
  return no_throw([&] {
    return greedy_allocation_impl(params, n_mats, alpha, P_max, block_error, user, rows, cap,
                                  n_rows);
  });
}

int spax_allocation_at(const double* rows, int32_t n_rows, int32_t n_mats, double target,
                       double* p) {
  clear_error();
  if (!rows || !p) return fail(SPAX_ERR_NULL, "rows and p are required");
  if (n_rows < 1 || n_mats < 1) return fail(SPAX_ERR_PARAM, "need n_rows >= 1 and n_mats >= 1");
  if (!std::isfinite(target)) return fail(SPAX_ERR_PARAM, "target is not finite");
  const size_t w = 1 + (size_t)n_mats;
  int32_t pick = n_rows - 1;
  if (target <= 0) {
    for (int m = 0; m < n_mats; ++m) p[m] = 0.0;
    return SPAX_OK;
  }
  for (int32_t r = 0; r < n_rows; ++r)
    if (rows[r * w] >= target - 1e-12) {
      pick = r;
      break;
    }
  for (int m = 0; m < n_mats; ++m) p[m] = rows[pick * w + 1 + m];
  return SPAX_OK;
}

}  // extern "C"
