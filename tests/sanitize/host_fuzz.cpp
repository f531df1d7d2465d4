// Seeded fuzz of libcpa's host-side C ABI, built with AddressSanitizer and
// UBSan (Makefile in this directory): the attention planner and metadata
// validator over ragged query/sequence lengths, shapes and options (valid and
// not), the chunk-size predictor and the online calibration over random and
// non-finite coefficients, the token-budget batch former over random request
// streams, and the micro-batch split point. Besides the sanitizers' own
// checks, each call's status and outputs are held to what include/cpa.h
// promises, recomputed here by brute force where that is cheap.
//
//   host_fuzz [seed] [iterations]      exit status 0 = every check held
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <set>
#include <vector>

#include "cpa.h"

namespace {

std::mt19937_64 rng;
long checks = 0;

#define CHECK(cond, ...)                                                        \
  do {                                                                          \
    ++checks;                                                                   \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "host_fuzz: check failed at line %d: %s\n", __LINE__, \
                   #cond);                                                      \
      std::fprintf(stderr, __VA_ARGS__);                                        \
      std::fprintf(stderr, "\n");                                               \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

int64_t uni(int64_t lo, int64_t hi) {  // inclusive
  return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
}
bool coin(double p = 0.5) { return std::uniform_real_distribution<double>(0, 1)(rng) < p; }
template <class T>
T pick(std::initializer_list<T> v) {
  return *(v.begin() + uni(0, (int64_t)v.size() - 1));
}

double wild_double() {
  switch (uni(0, 9)) {
    case 0: return std::numeric_limits<double>::quiet_NaN();
    case 1: return std::numeric_limits<double>::infinity();
    case 2: return -std::numeric_limits<double>::infinity();
    case 3: return 0.0;
    case 4: return -std::ldexp(1.0, (int)uni(-40, 10));
    case 5: return 1e300;
    default: return std::ldexp(1.0 + std::uniform_real_distribution<double>(0, 1)(rng),
                               (int)uni(-40, 0));
  }
}

bool valid_status(cpa_status s) { return s <= 0 && s >= -5; }

// ---- planner --------------------------------------------------------------

void fuzz_plan() {
  cpa_layer_desc d{};
  const int G = (int)pick<int64_t>({1, 2, 4, 5, 8, 16});
  d.num_kv_heads = (int)pick<int64_t>({1, 2, 4, 8, 40});
  d.num_q_heads = d.num_kv_heads * G + (coin(0.05) ? 1 : 0);
  d.head_dim = coin(0.05) ? 96 : (coin() ? 64 : 128);
  d.page_size = coin(0.05) ? 100 : (int)(16 << uni(0, 6));
  d.max_blocks_per_seq = (int)uni(coin(0.03) ? -1 : 1, 300);
  d.num_blocks = (int)uni(coin(0.03) ? 0 : 1, 5000);
  d.scale = coin(0.03) ? NAN : 1.0f / std::sqrt((float)d.head_dim);
  d.out_dtype = coin(0.03) ? 7 : (int)uni(0, 1);
  const int S = (int)uni(0, 40);
  std::vector<int32_t> ql(S), sl(S);
  const int64_t maxlen = (int64_t)d.max_blocks_per_seq * d.page_size;
  for (int s = 0; s < S; ++s) {
    const int kind = (int)uni(0, 9);
    // mostly up to 16k tokens; now and then up to the table's limit
    const int64_t cap = coin(0.05) ? maxlen : std::min<int64_t>(maxlen, 16384);
    int64_t n = kind == 0 ? uni(0, 4) : uni(0, std::max<int64_t>(0, cap));
    if (coin(0.02)) n = maxlen + uni(1, 100);              // too long for the table
    sl[s] = (int32_t)n;
    ql[s] = (int32_t)(kind < 3 ? std::min<int64_t>(n, 1) : uni(0, n));
    if (coin(0.02)) ql[s] = (int32_t)(n + 1);                // query_len > seq_len
    if (coin(0.01)) ql[s] = -1;
  }
  cpa_plan_options opt{};
  const bool use_opt = coin(0.6);
  if (use_opt) {
    opt.target_items = (int)uni(coin(0.02) ? -1 : 0, 600);
    opt.num_cus = (int)uni(0, 400);
    opt.prefill_split = coin(0.3) ? (int)uni(0, 9) : 0;
    // tiny decode splits make plans of up to the item limit: rare, as each
    // costs seconds under the sanitizers
    opt.decode_split_keys = coin(0.3) ? (int)(coin(0.03) ? uni(1, 63) : uni(64, 3000)) : 0;
    opt.min_split_keys = coin(0.3) ? (int)(64 * uni(0, 40)) + (coin(0.05) ? 7 : 0) : 0;
  }
  cpa_plan plan = nullptr;
  size_t ws = 0;
  const cpa_status st =
      cpa_plan_create(&d, S ? ql.data() : nullptr, S ? sl.data() : nullptr, S,
                      use_opt ? &opt : nullptr, &plan, &ws);
  CHECK(valid_status(st), "status %d", st);
  if (st != CPA_OK) {
    CHECK(plan == nullptr, "failed plan_create left a plan");
    CHECK(cpa_last_error()[0] != '\0', "failed call left no message");
    return;
  }
  // A plan was accepted: the inputs must have been valid.
  int64_t total = 0, pairs = 0;
  for (int s = 0; s < S; ++s) {
    CHECK(ql[s] >= 0 && ql[s] <= sl[s], "accepted query_len %d seq_len %d", ql[s], sl[s]);
    CHECK((sl[s] + d.page_size - 1) / d.page_size <= d.max_blocks_per_seq, "too many pages");
    total += ql[s];
    const int64_t h = sl[s] - ql[s];
    pairs += (int64_t)d.num_q_heads * (ql[s] * h + (int64_t)ql[s] * (ql[s] + 1) / 2);
  }
  cpa_plan_info info{};
  CHECK(cpa_plan_get_info(plan, &info) == CPA_OK, "get_info");
  CHECK(info.num_tokens == total, "tokens %d vs %" PRId64, info.num_tokens, total);
  CHECK(info.num_seqs == S, "seqs");
  CHECK(info.visible_pairs == pairs, "pairs %" PRId64 " vs %" PRId64, info.visible_pairs, pairs);
  CHECK(info.workspace_bytes == ws && ws >= 256 && ws % 256 == 0, "workspace %zu", ws);
  CHECK(info.num_prefill_items >= 0 && info.num_decode_items >= 0, "item counts");
  CHECK((info.num_combine_items == 0) == (info.num_partial_rows == 0), "combine vs partials");
  if (total == 0) CHECK(info.num_prefill_items + info.num_decode_items == 0, "items, no tokens");
  // NULL-pointer checks of the calls that would queue GPU work
  CHECK(cpa_attention(plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
            (total ? CPA_ERR_INVALID_ARG : CPA_OK), "attention NULL");
  CHECK(cpa_plan_upload(plan, nullptr, ws, nullptr) == CPA_ERR_INVALID_ARG, "upload NULL");
  CHECK(cpa_plan_destroy(plan) == CPA_OK, "destroy");
}

// ---- metadata validator ---------------------------------------------------

void fuzz_validate() {
  cpa_layer_desc d{4, 2, 64, (int)(16 << uni(0, 3)), (int)uni(1, 64), (int)uni(1, 16), 0.125f, 0};
  const int T = (int)uni(0, 200);
  const int64_t slots = (int64_t)d.num_blocks * d.page_size;
  std::vector<int32_t> sm(T);
  for (auto& x : sm) x = (int32_t)(coin(0.1) ? -uni(1, 5) : uni(0, slots - 1 + (coin(0.05) ? 3 : 0)));
  bool ok = true;
  std::set<int32_t> seen;
  for (int32_t x : sm) {
    if (x < 0) continue;
    if (x >= slots || !seen.insert(x).second) ok = false;
  }
  const cpa_status st = cpa_validate_metadata(&d, T ? sm.data() : nullptr, T, nullptr, nullptr,
                                              nullptr, 0);
  CHECK(st == (ok ? CPA_OK : CPA_ERR_INVALID_ARG), "slot check %d expected %d", st, ok);
  // block tables
  const int S = (int)uni(1, 6);
  std::vector<int32_t> ql(S), sl(S), bt((size_t)S * d.max_blocks_per_seq);
  for (int s = 0; s < S; ++s) {
    sl[s] = (int32_t)uni(0, (int64_t)d.max_blocks_per_seq * d.page_size);
    ql[s] = (int32_t)uni(0, sl[s]);
  }
  bool bok = true;
  for (int s = 0; s < S; ++s)
    for (int j = 0; j < d.max_blocks_per_seq; ++j) {
      int32_t v = (int32_t)uni(0, d.num_blocks - 1);
      if (coin(0.02)) v = coin() ? -1 : d.num_blocks;
      bt[(size_t)s * d.max_blocks_per_seq + j] = v;
      if (j < (sl[s] + d.page_size - 1) / d.page_size && (v < 0 || v >= d.num_blocks)) bok = false;
    }
  const cpa_status st2 = cpa_validate_metadata(&d, nullptr, 0, bt.data(), ql.data(), sl.data(), S);
  CHECK(st2 == (bok ? CPA_OK : CPA_ERR_INVALID_ARG), "block table check %d expected %d", st2, bok);
}

// ---- predictor and calibration -------------------------------------------

cpa_predictor_cfg random_cfg() {
  cpa_predictor_cfg c{};
  c.base_chunk_size = pick<int64_t>({2048, 512, 4096, 1});
  c.align = pick<int64_t>({128, 16, 1, 64, 0});
  c.min_chunk = pick<int64_t>({64, 0, 1, 256});
  c.max_chunk = pick<int64_t>({2048, 8192, 64, 0});
  c.max_model_len = pick<int64_t>({32768, 4096, 100000});
  c.smooth_factor = coin(0.8) ? 1.0 : wild_double();
  return c;
}

void fuzz_predictor() {
  int64_t sizes[80];
  const int n = (int)uni(-2, 80);
  const int64_t base = uni(-5, 5000), lo = uni(-5, 100);
  const cpa_status st = cpa_predictor_profile_sizes(base, n, lo, sizes);
  CHECK(valid_status(st), "profile sizes status");
  if (st == CPA_OK)
    for (int i = 0; i < n; ++i) {
      CHECK(sizes[i] <= base && sizes[i] >= lo, "size %" PRId64, sizes[i]);
      if (i) CHECK(sizes[i] < sizes[i - 1], "sizes not decreasing");
    }
  // fit over random, partly degenerate data
  const int m = (int)uni(0, 70);
  std::vector<double> l(m), t(m);
  for (int i = 0; i < m; ++i) {
    l[i] = coin(0.1) ? 5.0 : (double)uni(1, 4096);
    t[i] = coin(0.03) ? wild_double() : 1e-3 * l[i] + 1e-7 * l[i] * l[i];
  }
  double a = 0, b = 0, c = 0;
  const cpa_status fs = cpa_predictor_fit(m ? l.data() : nullptr, m ? t.data() : nullptr, m, &a, &b, &c);
  CHECK(valid_status(fs), "fit status");
  if (fs == CPA_OK) CHECK(std::isfinite(a) && std::isfinite(b) && std::isfinite(c), "fit non-finite");
  // chunk solve
  for (int k = 0; k < 20; ++k) {
    const cpa_predictor_cfg cfg = random_cfg();
    a = wild_double();
    b = wild_double();
    double T = 0;
    const cpa_status ts = cpa_predictor_target(&cfg, a, b, &T);
    CHECK(valid_status(ts), "target status");
    if (coin(0.3)) T = wild_double();
    const int64_t L = uni(-2, 40000), rem = uni(-2, 40000);
    int64_t chunk = -99;
    double x = 0;
    const cpa_status cs = cpa_predictor_next_chunk(&cfg, a, b, T, L, rem, &chunk, coin() ? &x : nullptr);
    CHECK(valid_status(cs), "next_chunk status");
    if (cs == CPA_OK) {
      CHECK(chunk >= 0, "negative chunk");
      CHECK(chunk <= std::max<int64_t>(0, rem), "chunk %" PRId64 " > remaining %" PRId64, chunk, rem);
      CHECK(chunk <= std::max<int64_t>(0, cfg.max_chunk), "chunk above max_chunk");
      CHECK(chunk <= std::max<int64_t>(0, cfg.max_model_len - L), "chunk past max_model_len");
    }
    double c2 = wild_double(), T2 = 0;
    if (cpa_calib_target(&cfg, a, b, c2, &T2) != CPA_OK) T2 = wild_double();
    const cpa_status ks = cpa_calib_next_chunk(&cfg, a, b, c2, T2, L, rem, &chunk, &x);
    CHECK(valid_status(ks), "calib next_chunk status");
    if (ks == CPA_OK) CHECK(chunk >= 0 && chunk <= std::max<int64_t>(0, rem), "calib chunk");
  }
}

void fuzz_calib() {
  cpa_calib cal = nullptr;
  const int minp = (int)uni(0, 12), win = (int)uni(0, 40);
  const cpa_status st = cpa_calib_create(minp, win, &cal);
  CHECK(valid_status(st), "calib create");
  if (st != CPA_OK) {
    CHECK(cal == nullptr, "failed create left an object");
    return;
  }
  const int recs = (int)uni(0, 80);
  for (int i = 0; i < recs; ++i) {
    const int n = (int)uni(0, 5);
    std::vector<int32_t> C(n), H(n);
    for (int j = 0; j < n; ++j) {
      C[j] = (int32_t)(coin(0.5) ? 512 : uni(0, 2048));
      H[j] = (int32_t)uni(coin(0.02) ? -3 : 0, 30000);
    }
    double feat[3];
    const cpa_status fs = cpa_calib_features(n ? C.data() : nullptr, n ? H.data() : nullptr, n, feat);
    CHECK(valid_status(fs), "features status");
    if (fs != CPA_OK) continue;
    int32_t ready = -1;
    const double ms = coin(0.05) ? wild_double() : 1e-3 * (1 + feat[0] * 1e-7);
    CHECK(valid_status(cpa_calib_record(cal, feat, ms, coin() ? &ready : nullptr)), "record");
    double a, b, c;
    int32_t pts = 0;
    const cpa_status ms_ = cpa_calib_model(cal, &a, &b, &c, &pts);
    CHECK(valid_status(ms_), "model status");
    if (ms_ == CPA_OK) CHECK(pts >= minp && pts <= win, "points %d", pts);
  }
  CHECK(cpa_calib_destroy(cal) == CPA_OK, "calib destroy");
}

// ---- batch former ----------------------------------------------------------

void fuzz_sched() {
  cpa_sched_cfg cfg{};
  cfg.budget = (int32_t)uni(coin(0.03) ? 0 : 1, 4096);
  cfg.rule = (int32_t)uni(0, coin(0.03) ? 5 : 3);
  cfg.fixed_chunk = (int32_t)uni(0, 2048);
  cfg.num_sizes = (int32_t)uni(0, 9);
  for (int i = 0; i < 8; ++i) cfg.sizes[i] = (int32_t)uni(0, 2048);
  cfg.pred = random_cfg();
  cfg.a = coin(0.8) ? 1e-8 : wild_double();
  cfg.b = coin(0.8) ? 1e-5 : wild_double();
  cfg.c = coin(0.8) ? 1e-2 : wild_double();
  cfg.T = coin(0.8) ? 0.05 : wild_double();
  cpa_sched s = nullptr;
  const cpa_status st = cpa_sched_create(&cfg, &s);
  CHECK(valid_status(st), "sched create");
  if (st != CPA_OK) return;
  const int R = (int)uni(0, 12);
  int64_t want_tokens = 0;
  for (int r = 0; r < R; ++r) {
    int32_t id = -1;
    const int32_t p = (int32_t)uni(coin(0.03) ? -1 : 1, 3000), mn = (int32_t)uni(0, 20);
    const cpa_status as = cpa_sched_add(s, p, mn, (int32_t)uni(0, 10), &id);
    CHECK(valid_status(as), "add status");
    if (as == CPA_OK) want_tokens += (int64_t)p + mn;
  }
  int64_t got_tokens = 0;
  for (int step = 0; step < 5000; ++step) {
    int32_t done = 0, k = 0;
    CHECK(cpa_sched_status(s, &done, &k) == CPA_OK, "status");
    if (done) break;
    int32_t cap = (int32_t)uni(0, 16), ns = 0;
    std::vector<int32_t> ids(64), q(64), n(64);
    cpa_status fs = cpa_sched_form(s, cap, ids.data(), q.data(), n.data(), &ns);
    if (fs == CPA_ERR_INVALID_ARG) {
      CHECK(ns > cap && ns <= 64, "needed %d of capacity %d", ns, cap);
      fs = cpa_sched_form(s, ns, ids.data(), q.data(), n.data(), &ns);
    }
    CHECK(fs == CPA_OK, "form %d", fs);
    int64_t tok = 0;
    for (int i = 0; i < ns; ++i) {
      CHECK(q[i] >= 1 && q[i] <= n[i], "row %d: q %d n %d", i, q[i], n[i]);
      tok += q[i];
    }
    CHECK(tok <= cfg.budget, "step over budget: %" PRId64 " > %d", tok, cfg.budget);
    got_tokens += tok;
    CHECK(cpa_sched_commit(s) == CPA_OK, "commit");
  }
  int32_t done = 0, k = 0;
  cpa_sched_status(s, &done, &k);
  if (done) CHECK(got_tokens == want_tokens, "tokens %" PRId64 " vs %" PRId64, got_tokens, want_tokens);
  CHECK(cpa_sched_destroy(s) == CPA_OK, "sched destroy");
}

// ---- micro-batch split ------------------------------------------------------

void fuzz_split() {
  const int S = (int)uni(0, 30);
  std::vector<int32_t> ql(S);
  for (auto& x : ql) x = (int32_t)(coin(0.02) ? -1 : uni(0, 3000));
  int32_t ss = -1, ts = -1;
  const int mode = (int)uni(0, coin(0.05) ? 4 : 1);
  const cpa_status st = cpa_split_point(S ? ql.data() : nullptr, S, mode, coin(0.05) ? -1.0 : 0.5,
                                        (int32_t)uni(0, 500), &ss, &ts);
  CHECK(valid_status(st), "split status");
  if (st != CPA_OK) return;
  CHECK(ss >= 0 && ss < std::max(1, S), "seq split %d of %d", ss, S);
  int64_t pre = 0;
  for (int i = 0; i < ss; ++i) pre += ql[i];
  CHECK(ts == pre, "token split %d vs %" PRId64, ts, pre);
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const long iters = argc > 2 ? std::strtol(argv[2], nullptr, 10) : 2000;
  rng.seed(seed);
  for (long i = 0; i < iters; ++i) {
    fuzz_plan();
    fuzz_validate();
    if (i % 4 == 0) fuzz_predictor();
    if (i % 8 == 0) fuzz_calib();
    if (i % 8 == 4) fuzz_sched();
    fuzz_split();
  }
  std::printf("host_fuzz: seed %" PRIu64 ", %ld iterations, %ld checks passed\n", seed, iters, checks);
  return 0;
}
