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
#include <new>
#include <string>
#include <vector>

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

// Householder QR least squares for an n x 3 system; A is column-major
// (column j at A[j*n]) and is overwritten, as is y.
bool lstsq3(double* A, double* y, int n, double coef[3]) {
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

// Post-processing shared by both models: smoothing with smooth_factor,
// floor(xs + 1e-6), alignment down, min_chunk, then the caps.
int64_t finish_chunk(const cpa_predictor_cfg* cfg, double x, int64_t history_len,
                     int64_t remaining) {
  const int64_t base = cfg->base_chunk_size;
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
  return out;
}

// Positive root C of a*C^2 + (a*H + b)*C + (b*H + c - T) = 0 (the
// two-variable model f(C,H) = T), with the fallbacks stated in cpa.h.
double raw_root2(double a, double b, double c, double T, int64_t H, int64_t base) {
  const bool fin = std::isfinite(a) && std::isfinite(b) && std::isfinite(c) && std::isfinite(T);
  const double h = (double)H;
  if (a > 0 && fin) {
    const double B = a * h + b;
    const double K = b * h + c - T;
    const double disc = B * B - 4.0 * a * K;
    if (disc >= 0.0) return (-B + std::sqrt(disc)) / (2.0 * a);
    return (double)base;
  }
  if (fin) {
    const double B = a * h + b;
    if (B > 0) return (T - b * h - c) / B;
  }
  return (double)base;
}

// Least squares for ms ~ a*F0 + b*F1 + c*F2, columns scaled by their
// largest magnitude.
cpa_status fit_features(const double* feats, const double* ms, int32_t n, double out[3]) {
  if (n < 3) return cpa::fail(CPA_ERR_INVALID_ARG, "calib fit: need at least 3 records");
  double scale[3] = {0.0, 0.0, 0.0};
  for (int32_t i = 0; i < n; ++i) {
    for (int j = 0; j < 3; ++j) {
      const double v = feats[(size_t)i * 3 + j];
      if (!std::isfinite(v))
        return cpa::fail(CPA_ERR_NUMERIC, "calib fit: non-finite feature " + std::to_string(i));
      scale[j] = std::fmax(scale[j], std::fabs(v));
    }
    if (!std::isfinite(ms[i]))
      return cpa::fail(CPA_ERR_NUMERIC, "calib fit: non-finite time " + std::to_string(i));
  }
  for (int j = 0; j < 3; ++j)
    if (!(scale[j] > 0.0)) return cpa::fail(CPA_ERR_NUMERIC, "calib fit: a feature column is zero");
  std::basic_string<double> A((size_t)n * 3, 0.0), y(ms, ms + n);
  for (int32_t i = 0; i < n; ++i)
    for (int j = 0; j < 3; ++j) A[(size_t)j * n + i] = feats[(size_t)i * 3 + j] / scale[j];
  double coef[3];
  if (!lstsq3(A.data(), y.data(), n, coef))
    return cpa::fail(CPA_ERR_NUMERIC, "calib fit: records do not determine three coefficients");
  for (int j = 0; j < 3; ++j) out[j] = coef[j] / scale[j];
  return cpa::ok();
}

}  // namespace

extern "C" cpa_status cpa_predictor_profile_sizes(int64_t base, int32_t n, int64_t lo,
                                                  int64_t* sizes) {
  if (!sizes || n < 2 || lo < 1 || base <= lo)
    return cpa::fail(CPA_ERR_INVALID_ARG, "profile_sizes: need n >= 2, base > lo >= 1");
  // n distinct sizes need a spacing of at least one token (with a spacing of
  // exactly one every size is an integer, so the rounding merges none)
  if (base - lo < (int64_t)n - 1)
    return cpa::fail(CPA_ERR_INVALID_ARG, "profile_sizes: base - lo < n - 1 cannot give n "
                                          "distinct sizes");
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
  std::basic_string<double> A((size_t)n * 3, 0.0), y(ms, ms + n);
  for (int32_t i = 0; i < n; ++i) {
    const double u = lens[i] / scale;
    A[i] = u * u;
    A[(size_t)n + i] = u;
    A[(size_t)2 * n + i] = 1.0;
  }
  double coef[3];
  if (!lstsq3(A.data(), y.data(), n, coef))
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
  const int64_t out = finish_chunk(cfg, x, history_len, remaining);
  *chunk = out;
  if (raw_x) *raw_x = x;
  return cpa::ok();
}

// ---- Online calibration: [CPP] "online calibration" ----

extern "C" cpa_status cpa_calib_features(const int32_t* chunk_lens, const int32_t* hist_lens,
                                         int32_t n, double* feat) {
  if (!feat || n < 0 || (n > 0 && (!chunk_lens || !hist_lens)))
    return cpa::fail(CPA_ERR_INVALID_ARG, "calib_features: bad arguments");
  double f0 = 0.0, f1 = 0.0, cnt = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    if (chunk_lens[i] <= 0) continue;
    if (hist_lens[i] < 0) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_features: negative history");
    const double C = (double)chunk_lens[i], CH = (double)((int64_t)chunk_lens[i] + hist_lens[i]);
    f0 += C * CH;
    f1 += CH;
    cnt += 1.0;
  }
  feat[0] = f0;
  feat[1] = f1;
  feat[2] = cnt;
  return cpa::ok();
}

extern "C" cpa_status cpa_calib_fit(const double* feats, const double* ms, int32_t n, double* a,
                                    double* b, double* c) {
  if (!feats || !ms || !a || !b || !c) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_fit: null pointer");
  double out[3];
  const cpa_status st = fit_features(feats, ms, n, out);
  if (st != CPA_OK) return st;
  *a = out[0];
  *b = out[1];
  *c = out[2];
  return cpa::ok();
}

extern "C" cpa_status cpa_calib_target(const cpa_predictor_cfg* cfg, double a, double b, double c,
                                       double* T) {
  if (!cfg || !T) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_target: null pointer");
  const double base = (double)cfg->base_chunk_size;
  *T = a * base * base + b * base + c;
  return cpa::ok();
}

extern "C" cpa_status cpa_calib_next_chunk(const cpa_predictor_cfg* cfg, double a, double b,
                                           double c, double T, int64_t history_len,
                                           int64_t remaining, int64_t* chunk, double* raw_x) {
  if (!cfg || !chunk) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_next_chunk: null pointer");
  if (cfg->align <= 0 || cfg->base_chunk_size <= 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "calib_next_chunk: align and base_chunk_size must be > 0");
  const double x = raw_root2(a, b, c, T, history_len, cfg->base_chunk_size);
  *chunk = finish_chunk(cfg, x, history_len, remaining);
  if (raw_x) *raw_x = x;
  return cpa::ok();
}

// Record window: the most recent `window` records, refitted after each
// record once min_points are held.
struct cpa_calib_s {
  int32_t min_points = 5, window = 30;
  std::vector<double> feats;  // ring of window x 3
  std::vector<double> ms;     // ring of window
  int32_t count = 0;          // records held (<= window)
  int32_t next = 0;           // ring slot of the next record
  bool ready = false;
  double coef[3] = {0.0, 0.0, 0.0};
};

extern "C" cpa_status cpa_calib_create(int32_t min_points, int32_t window, cpa_calib* out) {
  if (!out) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_create: null pointer");
  *out = nullptr;
  if (min_points < 3 || window < min_points)
    return cpa::fail(CPA_ERR_INVALID_ARG, "calib_create: need 3 <= min_points <= window");
  cpa_calib_s* h = new (std::nothrow) cpa_calib_s;
  if (!h) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_create: out of host memory");
  h->min_points = min_points;
  h->window = window;
  h->feats.assign((size_t)window * 3, 0.0);
  h->ms.assign((size_t)window, 0.0);
  *out = h;
  return cpa::ok();
}

extern "C" cpa_status cpa_calib_destroy(cpa_calib h) {
  delete h;
  return cpa::ok();
}

extern "C" cpa_status cpa_calib_record(cpa_calib h, const double* feat, double ms,
                                       int32_t* ready) {
  if (!h || !feat) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_record: null pointer");
  for (int j = 0; j < 3; ++j) h->feats[(size_t)h->next * 3 + j] = feat[j];
  h->ms[h->next] = ms;
  h->next = (h->next + 1) % h->window;
  if (h->count < h->window) ++h->count;
  cpa_status st = CPA_OK;
  if (h->count >= h->min_points) {
    // Oldest first, as the records arrived.
    std::vector<double> f((size_t)h->count * 3), t((size_t)h->count);
    const int32_t first = (h->next - h->count + h->window) % h->window;
    for (int32_t i = 0; i < h->count; ++i) {
      const int32_t slot = (first + i) % h->window;
      for (int j = 0; j < 3; ++j) f[(size_t)i * 3 + j] = h->feats[(size_t)slot * 3 + j];
      t[i] = h->ms[slot];
    }
    double out[3];
    st = fit_features(f.data(), t.data(), h->count, out);
    if (st == CPA_OK) {
      for (int j = 0; j < 3; ++j) h->coef[j] = out[j];
      h->ready = true;
    }
  }
  if (ready) *ready = h->ready ? 1 : 0;
  return st;
}

extern "C" cpa_status cpa_calib_model(cpa_calib h, double* a, double* b, double* c,
                                      int32_t* points) {
  if (!h || !a || !b || !c) return cpa::fail(CPA_ERR_INVALID_ARG, "calib_model: null pointer");
  if (points) *points = h->count;
  if (!h->ready) return cpa::fail(CPA_ERR_NUMERIC, "calib_model: fewer records than min_points");
  *a = h->coef[0];
  *b = h->coef[1];
  *c = h->coef[2];
  return cpa::ok();
}
