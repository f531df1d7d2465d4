// Threaded driver of the host half of libcpa for the ThreadSanitizer build:
// eight threads at once create, inspect, upload and destroy plans (their
// uploads share one process-wide workspace registry), call the attention
// entry point until its (stubbed) launch fails, hit refusals whose messages
// are per thread, and run the predictor, the online calibration and the
// batch former on objects of their own. Exits non-zero on a wrong result;
// the sanitizer reports any data race.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "cpa.h"

namespace {

bool fail(const char* what) {
  std::fprintf(stderr, "FAIL %s (%s)\n", what, cpa_last_error());
  return false;
}

bool worker(int id, int iters, void* shared_ws, size_t ws_bytes) {
  const cpa_layer_desc desc = {32, 8, 128, 128, 200, 104, 0.0883883f, 0};
  cpa_layer_desc bad = desc;
  bad.head_dim = 96;
  const int32_t ql[3] = {512, 1, 40 + id};
  const int32_t sl[3] = {12800, 700, 300 + id};
  // A private workspace per thread, and the shared one that every thread
  // uploads to in turn (the registry keeps the last uploader's plan).
  std::vector<unsigned char> mine(ws_bytes + 256);
  void* own = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(mine.data()) + 255) & ~uintptr_t(255));
  const cpa_predictor_cfg cfg = {2048, 128, 64, 2048, 32768, 1.0};
  for (int i = 0; i < iters; ++i) {
    cpa_plan plan = nullptr;
    size_t ws = 0;
    if (cpa_plan_create(&desc, ql, sl, 3, nullptr, &plan, &ws) != CPA_OK) return fail("plan_create");
    cpa_plan_info info;
    if (cpa_plan_get_info(plan, &info) != CPA_OK || info.num_tokens != 553 + id ||
        info.workspace_bytes != ws || ws > ws_bytes)
      return fail("plan_info");
    if (cpa_plan_upload(plan, own, ws_bytes, nullptr) != CPA_OK) return fail("upload own");
    if (cpa_plan_upload(plan, shared_ws, ws_bytes, nullptr) != CPA_OK) return fail("upload shared");
    // The launch is stubbed out: the call must fail with CPA_ERR_HIP, after
    // the checks that read the registry.
    static const uint16_t dummy[16] = {};
    void* out = own;
    if (cpa_attention(plan, dummy, dummy, dummy, reinterpret_cast<const int32_t*>(dummy), out,
                      own, ws_bytes, nullptr) != CPA_ERR_HIP)
      return fail("attention on own workspace");
    if (cpa_plan_destroy(plan) != CPA_OK) return fail("plan_destroy");
    cpa_plan p2 = nullptr;
    if (cpa_plan_create(&bad, ql, sl, 3, nullptr, &p2, &ws) != CPA_ERR_UNSUPPORTED || p2)
      return fail("refusal");
    if (std::strstr(cpa_last_error(), "head_dim") == nullptr) return fail("refusal message");

    int64_t chunk = 0;
    double raw = 0;
    if (cpa_predictor_next_chunk(&cfg, 2e-9, 5e-6, 0.0125, 4096 + id, 30000, &chunk, &raw) !=
            CPA_OK ||
        chunk <= 0 || chunk > 2048)
      return fail("next_chunk");

    cpa_calib cal = nullptr;
    if (cpa_calib_create(5, 30, &cal) != CPA_OK) return fail("calib_create");
    for (int k = 0; k < 12; ++k) {
      const int32_t c = 128 * (k + 1), h = 256 * k;
      double feat[3];
      if (cpa_calib_features(&c, &h, 1, feat) != CPA_OK) return fail("features");
      const double ms = 1e-6 * feat[0] + 1e-4 * feat[1] + 0.01 * feat[2];
      if (cpa_calib_record(cal, feat, ms, nullptr) != CPA_OK) return fail("record");
    }
    double a, b, c;
    if (cpa_calib_model(cal, &a, &b, &c, nullptr) != CPA_OK || std::fabs(a - 1e-6) > 1e-12)
      return fail("calib_model");
    cpa_calib_destroy(cal);

    cpa_sched_cfg sc;
    std::memset(&sc, 0, sizeof sc);
    sc.budget = 512;
    sc.rule = CPA_RULE_FIXED;
    sc.fixed_chunk = 256;
    cpa_sched s = nullptr;
    if (cpa_sched_create(&sc, &s) != CPA_OK) return fail("sched_create");
    int32_t rid;
    cpa_sched_add(s, 1000 + id, 2, 0, &rid);
    cpa_sched_add(s, 300, 1, 0, &rid);
    int32_t ids[16], q[16], n[16], cnt = 0, fin = 0, step = 0;
    while (!fin) {
      if (cpa_sched_form(s, 16, ids, q, n, &cnt) != CPA_OK || cpa_sched_commit(s) != CPA_OK)
        return fail("sched step");
      if (cpa_sched_status(s, &fin, &step) != CPA_OK || step > 100) return fail("sched status");
    }
    cpa_sched_destroy(s);
  }
  return true;
}

}  // namespace

int main() {
  const size_t ws_bytes = 64u << 20;
  void* shared = std::aligned_alloc(256, ws_bytes);
  std::vector<std::thread> th;
  std::vector<int> ok(8, 0);
  for (int t = 0; t < 8; ++t)
    th.emplace_back([&, t] { ok[t] = worker(t, 40, shared, ws_bytes) ? 1 : 0; });
  for (auto& t : th) t.join();
  std::free(shared);
  for (int t = 0; t < 8; ++t)
    if (!ok[t]) return 1;
  std::printf("host threads ok\n");
  return 0;
}
