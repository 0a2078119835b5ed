// Host-side helpers of libspax: errors, layout derivation, threshold/count conversions.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"

namespace spax {

static thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }

int hip_fail(hipError_t e, const char* what) {
  return fail(SPAX_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

static int64_t roundup(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool layout_ok(const spax_layout* L) {
  if (!L || L->n_mats < 1 || L->n_mats > SPAX_MAX_MATS || L->d_in < 1) return false;
  int64_t t = 0;
  for (int m = 0; m < L->n_mats; ++m) t += L->d_out[m];
  if (t != L->d_out_total || t <= 0) return false;
  if (L->stride_F <= 0 || L->stride_A <= 0 || L->stride_F % SPAX_RECORD_ALIGN ||
      L->stride_A % SPAX_RECORD_ALIGN)
    return false;
  if (L->off_A != (int64_t)L->d_in * L->stride_F) return false;
  if (L->total_bytes != L->off_A + (int64_t)L->d_in * L->stride_A) return false;
  return true;
}

// fp16 bit pattern (non-negative, <= 0x7C00) -> exact double value.
static double half_value(int32_t k) {
  int e = k >> 10, m = k & 0x3FF;
  if (e == 0) return std::ldexp((double)m, -24);
  if (e == 31) return INFINITY;
  return std::ldexp(1.0 + m / 1024.0, e - 15);
}

int tier_args_from_params(const spax_tier_params* p, int32_t d, TierArgs* out) {
  if (!p) return fail(SPAX_ERR_NULL, "tier params is NULL");
  TierArgs a{};
  a.mode = p->mode;
  a.d = d;
  a.k_full = a.k_skip = a.k_tau = 0;
  a.num = 0;
  a.den = 1;
  switch (p->mode) {
    case SPAX_MODE_TOPK:
      if (p->n_full < 0 || p->n_approx < 0 || (int64_t)p->n_full + p->n_approx > d)
        return fail(SPAX_ERR_PARAM, "TOPK counts (%d, %d) out of range for d=%d", p->n_full,
                    p->n_approx, d);
      a.n_full = p->n_full;
      a.n_approx = p->n_approx;
      break;
    case SPAX_MODE_THRESHOLD:
      if (std::isnan(p->tau_skip) || std::isnan(p->tau_full))
        return fail(SPAX_ERR_PARAM, "THRESHOLD tau is NaN");
      if (p->tau_skip > p->tau_full)
        return fail(SPAX_ERR_PARAM, "tau_skip %g > tau_full %g", p->tau_skip, p->tau_full);
      a.k_skip = spax_key_threshold(p->tau_skip);
      a.k_full = spax_key_threshold(p->tau_full);
      break;
    case SPAX_MODE_TOPK_GUIDED:
      if (std::isnan(p->tau)) return fail(SPAX_ERR_PARAM, "TOPK_GUIDED tau is NaN");
      if (p->n_skip_lo < 0 || p->n_skip_lo > p->n_skip_hi || p->n_skip_hi > d)
        return fail(SPAX_ERR_PARAM, "skip band [%d, %d] invalid for d=%d", p->n_skip_lo,
                    p->n_skip_hi, d);
      if (p->approx_den <= 0 || p->approx_den > 65535 || p->approx_num < 0 ||
          p->approx_num > p->approx_den)
        return fail(SPAX_ERR_PARAM, "approx split %d/%d invalid", p->approx_num, p->approx_den);
      a.k_tau = spax_key_threshold(p->tau);
      a.n_lo = p->n_skip_lo;
      a.n_hi = p->n_skip_hi;
      a.num = p->approx_num;
      a.den = p->approx_den;
      break;
    default:
      return fail(SPAX_ERR_PARAM, "unknown tier mode %d", p->mode);
  }
  *out = a;
  return SPAX_OK;
}

}  // namespace spax

using namespace spax;

extern "C" {

int spax_layout_init(spax_layout* L) {
  clear_error();
  if (!L) return fail(SPAX_ERR_NULL, "layout is NULL");
  if (L->n_mats < 1 || L->n_mats > SPAX_MAX_MATS)
    return fail(SPAX_ERR_SHAPE, "n_mats %d outside 1..%d", L->n_mats, SPAX_MAX_MATS);
  if (L->d_in < 1 || L->d_in > SPAX_MAX_DIN)
    return fail(SPAX_ERR_SHAPE, "d_in %d outside 1..%d", L->d_in, SPAX_MAX_DIN);
  if (L->base_fmt != SPAX_FMT_FP16 && L->base_fmt != SPAX_FMT_INT4)
    return fail(SPAX_ERR_SHAPE, "unknown base format %d", L->base_fmt);
  if (L->approx_group != 64 && L->approx_group != 128)
    return fail(SPAX_ERR_SHAPE, "approx_group %d not 64 or 128", L->approx_group);
  if (L->base_fmt == SPAX_FMT_INT4 && L->base_group != 128)
    return fail(SPAX_ERR_SHAPE, "int4 base_group %d not 128", L->base_group);
  int64_t t = 0;
  for (int m = 0; m < L->n_mats; ++m) {
    int32_t r = L->d_out[m];
    if (r <= 0 || r % L->approx_group || (L->base_fmt == SPAX_FMT_INT4 && r % L->base_group))
      return fail(SPAX_ERR_SHAPE, "d_out[%d] = %d is not a positive multiple of the group size",
                  m, r);
    t += r;
  }
  if (t > kMaxRowsTotal) return fail(SPAX_ERR_SHAPE, "d_out_total %lld too large", (long long)t);
  L->d_out_total = t;
  L->rec_F = L->base_fmt == SPAX_FMT_FP16 ? 2 * t : t / 2 + 4 * (t / L->base_group);
  L->rec_A = t / 4 + 4 * (t / L->approx_group);
  L->stride_F = roundup(L->rec_F, SPAX_RECORD_ALIGN);
  L->stride_A = roundup(L->rec_A, SPAX_RECORD_ALIGN);
  L->off_A = (int64_t)L->d_in * L->stride_F;
  L->total_bytes = L->off_A + (int64_t)L->d_in * L->stride_A;
  return SPAX_OK;
}

int32_t spax_key_threshold(double tau) {
  if (std::isnan(tau)) return -1;
  // half(k) is non-decreasing in k on [0, 0x7C00]: binary search the first k reaching tau.
  int32_t lo = 0, hi = 0x7C00;
  if (!(half_value(hi) >= tau)) return 0x7C01;
  while (lo < hi) {
    int32_t mid = (lo + hi) / 2;
    if (half_value(mid) >= tau) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

int spax_counts_from_fractions(int32_t d, double p_full, double p_approx, int32_t* n_full,
                               int32_t* n_approx) {
  clear_error();
  if (!n_full || !n_approx) return fail(SPAX_ERR_NULL, "output pointer is NULL");
  if (d < 0 || !std::isfinite(p_full) || !std::isfinite(p_approx) || p_full < 0 || p_approx < 0)
    return fail(SPAX_ERR_PARAM, "bad fractions");
  double nf = std::floor(p_full * d + 0.5);
  double nk = std::floor((p_full + p_approx) * d + 0.5);
  if (nf > d) nf = d;
  if (nk > d) nk = d;
  if (nk < nf) nk = nf;
  *n_full = (int32_t)nf;
  *n_approx = (int32_t)(nk - nf);
  return SPAX_OK;
}

int spax_guided_bounds(int32_t d, double s, double delta, int32_t* n_lo, int32_t* n_hi) {
  clear_error();
  if (!n_lo || !n_hi) return fail(SPAX_ERR_NULL, "output pointer is NULL");
  if (d < 0 || !std::isfinite(s) || !std::isfinite(delta) || delta < 0)
    return fail(SPAX_ERR_PARAM, "bad guided target");
  double lo = std::ceil(d * (s - delta) - 1e-9);
  double hi = std::floor(d * (s + delta) + 1e-9);
  if (lo < 0) lo = 0;
  if (hi > d) hi = d;
  *n_lo = (int32_t)lo;
  *n_hi = (int32_t)hi;
  return SPAX_OK;
}

const char* spax_status_string(int status) {
  switch (status) {
    case SPAX_OK: return "SPAX_OK";
    case SPAX_ERR_NULL: return "SPAX_ERR_NULL";
    case SPAX_ERR_SHAPE: return "SPAX_ERR_SHAPE";
    case SPAX_ERR_PARAM: return "SPAX_ERR_PARAM";
    case SPAX_ERR_ALIGN: return "SPAX_ERR_ALIGN";
    case SPAX_ERR_WORKSPACE: return "SPAX_ERR_WORKSPACE";
    case SPAX_ERR_HIP: return "SPAX_ERR_HIP";
    case SPAX_ERR_UNSUPPORTED: return "SPAX_ERR_UNSUPPORTED";
    case SPAX_ERR_HOST: return "SPAX_ERR_HOST";
    default: return "SPAX_ERR_UNKNOWN";
  }
}

const char* spax_last_error(void) { return g_err; }

const char* spax_version(void) { return "spax 0.1.0 (gfx950)"; }

}  // extern "C"
