// Chunk-size predictor (host, fp64). Built with -ffp-contract=off so every
// expression rounds exactly as written: the chunk sizes it returns are
// meant to be reproducible bit for bit by any IEEE-754 fp64 implementation
// that evaluates the same expressions in the same order.
//
// Source: vllm-ascend design "Dynamic chunked pipeline parallel (CPP)":
//   "quadratic latency model"  f(l) = a*l^2 + b*l + c;
//   "startup: profiling"       64 sizes from base_chunk_size to near zero,
//                              least-squares fit, target from the base size;
//   "runtime: dynamic prediction"
//                              T = f(base) - f(0); f(L+x) - f(L) = T expands
//                              to a*x^2 + (2aL+b)*x - T = 0, solved with the
//                              quadratic formula; smoothing, alignment down
//                              to a page multiple (at least 64), caps at
//                              max_model_len - history_len and the token cap.
#include <cmath>
#include <cstdint>
#include <string>

#include "cpa.h"
#include "cpa_host.h"

namespace {

constexpr double kEpsFloor = 1e-6;
constexpr double kXiCap = 9.0e15;

// Positive root of a*x^2 + (2aL+b)*x - T = 0, with the fallbacks stated in
// cpa.h for degenerate coefficients.
double raw_root(double a, double b, double T, int64_t L, int64_t base) {
  if (a > 0 && std::isfinite(a) && std::isfinite(b) && std::isfinite(T)) {
    const double B = 2.0 * a * (double)L + b;
    const double disc = B * B + 4.0 * a * T;
    if (disc >= 0.0) return (-B + std::sqrt(disc)) / (2.0 * a);
    return (double)base;
  }
  if (b > 0 && std::isfinite(b) && std::isfinite(T)) return T / b;
  return (double)base;
}

// Householder QR least squares for an n x 3 system (columns u^2, u, 1).
bool lstsq3(const double* u, const double* t, int n, double coef[3]) {
  // Column-major copy of the design and the right-hand side.
  std::basic_string<double> A((size_t)n * 3, 0.0), y(t, t + n);
  for (int i = 0; i < n; ++i) {
    A[i] = u[i] * u[i];
    A[n + i] = u[i];
    A[2 * n + i] = 1.0;
  }
  double rdiag[3];
  for (int k = 0; k < 3; ++k) {
    double* col = &A[(size_t)k * n];
    double norm = 0.0;
    for (int i = k; i < n; ++i) norm = std::hypot(norm, col[i]);
    if (!(norm > 0.0) || !std::isfinite(norm)) return false;
    if (col[k] > 0) norm = -norm;
    for (int i = k; i < n; ++i) col[i] /= -norm;
    col[k] += 1.0;
    for (int j = k + 1; j < 3; ++j) {
      double* cj = &A[(size_t)j * n];
      double s = 0.0;
      for (int i = k; i < n; ++i) s += col[i] * cj[i];
      s = -s / col[k];
      for (int i = k; i < n; ++i) cj[i] += s * col[i];
    }
    double s = 0.0;
    for (int i = k; i < n; ++i) s += col[i] * y[i];
    s = -s / col[k];
    for (int i = k; i < n; ++i) y[i] += s * col[i];
    rdiag[k] = norm;
  }
  // Back substitution with R (upper triangle above the diagonal in A).
  const double scale = std::fabs(rdiag[0]);
  for (int k = 2; k >= 0; --k) {
    if (std::fabs(rdiag[k]) <= 1e-12 * scale) return false;
    double s = y[k];
    for (int j = k + 1; j < 3; ++j) s -= A[(size_t)j * n + k] * coef[j];
    coef[k] = s / rdiag[k];
  }
  return true;
}

}  // namespace

extern "C" cpa_status cpa_predictor_profile_sizes(int64_t base, int32_t n, int64_t lo,
                                                  int64_t* sizes) {
  if (!sizes || n < 2 || lo < 1 || base <= lo)
    return cpa::fail(CPA_ERR_INVALID_ARG, "profile_sizes: need n >= 2, base > lo >= 1");
  for (int32_t i = 0; i < n; ++i) {
    const double v = (double)base - (double)i * (double)(base - lo) / (double)(n - 1);
    sizes[i] = (int64_t)std::nearbyint(v);
  }
  return cpa::ok();
}

extern "C" cpa_status cpa_predictor_fit(const double* lens, const double* ms, int32_t n,
                                        double* a, double* b, double* c) {
  if (!lens || !ms || !a || !b || !c) return cpa::fail(CPA_ERR_INVALID_ARG, "fit: null pointer");
  if (n < 3) return cpa::fail(CPA_ERR_INVALID_ARG, "fit: need at least 3 points");
  double scale = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    if (!std::isfinite(lens[i]) || !std::isfinite(ms[i]))
      return cpa::fail(CPA_ERR_NUMERIC, "fit: non-finite sample " + std::to_string(i));
    scale = std::fmax(scale, std::fabs(lens[i]));
  }
  if (!(scale > 0.0)) return cpa::fail(CPA_ERR_NUMERIC, "fit: all sizes are zero");
  std::basic_string<double> u((size_t)n, 0.0);
  for (int32_t i = 0; i < n; ++i) u[i] = lens[i] / scale;
  double coef[3];
  if (!lstsq3(u.data(), ms, n, coef))
    return cpa::fail(CPA_ERR_NUMERIC, "fit: sizes do not determine a quadratic");
  *a = coef[0] / (scale * scale);
  *b = coef[1] / scale;
  *c = coef[2];
  return cpa::ok();
}

extern "C" cpa_status cpa_predictor_target(const cpa_predictor_cfg* cfg, double a, double b,
                                           double* T) {
  if (!cfg || !T) return cpa::fail(CPA_ERR_INVALID_ARG, "target: null pointer");
  const double base = (double)cfg->base_chunk_size;
  *T = a * base * base + b * base;
  return cpa::ok();
}

extern "C" cpa_status cpa_predictor_next_chunk(const cpa_predictor_cfg* cfg, double a, double b,
                                               double T, int64_t history_len, int64_t remaining,
                                               int64_t* chunk, double* raw_x) {
  if (!cfg || !chunk) return cpa::fail(CPA_ERR_INVALID_ARG, "next_chunk: null pointer");
  if (cfg->align <= 0 || cfg->base_chunk_size <= 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "next_chunk: align and base_chunk_size must be > 0");
  const int64_t base = cfg->base_chunk_size;
  const double x = raw_root(a, b, T, history_len, base);
  const double s = cfg->smooth_factor;
  const double xs = s * x + (1.0 - s) * (double)base;
  const double xf = xs + kEpsFloor;
  int64_t xi;
  if (!(xf >= 0.0))
    xi = 0;
  else if (xf >= kXiCap)
    xi = (int64_t)kXiCap;
  else
    xi = (int64_t)std::floor(xf);
  int64_t xa = (xi / cfg->align) * cfg->align;
  if (xa < cfg->min_chunk) xa = cfg->min_chunk;
  int64_t out = xa;
  if (cfg->max_chunk < out) out = cfg->max_chunk;
  if (cfg->max_model_len - history_len < out) out = cfg->max_model_len - history_len;
  if (remaining < out) out = remaining;
  if (out < 0) out = 0;
  *chunk = out;
  if (raw_x) *raw_x = x;
  return cpa::ok();
}
