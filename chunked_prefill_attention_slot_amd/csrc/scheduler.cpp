// Token-budget batch former of chunked prefill (host).
//
// Source: the vLLM "Chunked-Prefills" article, section 3.1 (non-blocking
// scheduling under a token budget: decode requests first at one token each,
// then unfinished prefills, then new requests, each step within the budget),
// section 3.2.2 (fixed and progressive chunk sizes) and the vllm-ascend CPP
// design, "runtime: dynamic prediction" (the scheduler asks the predictor for
// the chunk size at the request's current prefix).
//
// The rules the pages leave open are stated with cpa_sched_form in cpa.h.
#include <algorithm>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "cpa.h"
#include "cpa_host.h"

namespace {

struct Req {
  int32_t prompt_len, max_new, arrival;
  int32_t prefilled = 0, generated = 0, chunks = 0;
  bool admitted = false;
  bool done() const { return prefilled == prompt_len && generated >= max_new; }
};

struct Entry {
  int32_t rid, q, n;
};

}  // namespace

struct cpa_sched_s {
  cpa_sched_cfg cfg;
  std::vector<Req> reqs;
  std::vector<int32_t> admitted;  // request ids in admission order
  std::vector<Entry> pending;
  bool formed = false;
  int32_t step = 0;
};

namespace {

// Chunk cap of the configured rule for a prefill at prefix L with `rem`
// prompt tokens left, the request's k-th chunk.
cpa_status cap_of(const cpa_sched_s* s, int32_t L, int32_t rem, int32_t k, int64_t* cap) {
  const cpa_sched_cfg& c = s->cfg;
  double x;
  switch (c.rule) {
    case CPA_RULE_FIXED:
      *cap = c.fixed_chunk;
      return cpa::ok();
    case CPA_RULE_PROGRESSIVE:
      *cap = c.sizes[std::min(k, c.num_sizes - 1)];
      return cpa::ok();
    case CPA_RULE_PREDICTOR:
      return cpa_predictor_next_chunk(&c.pred, c.a, c.b, c.T, L, rem, cap, &x);
    case CPA_RULE_CALIBRATED:
      return cpa_calib_next_chunk(&c.pred, c.a, c.b, c.c, c.T, L, rem, cap, &x);
    default:
      return cpa::fail(CPA_ERR_INVALID_ARG, "sched: unknown rule");
  }
}

}  // namespace

extern "C" cpa_status cpa_sched_create(const cpa_sched_cfg* cfg, cpa_sched* out) {
  if (!cfg || !out) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: null pointer");
  *out = nullptr;
  if (cfg->budget <= 0) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: budget must be > 0");
  if (cfg->rule < CPA_RULE_FIXED || cfg->rule > CPA_RULE_CALIBRATED)
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: unknown rule");
  if (cfg->rule == CPA_RULE_FIXED && cfg->fixed_chunk <= 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: fixed_chunk must be > 0");
  if (cfg->rule == CPA_RULE_PROGRESSIVE) {
    if (cfg->num_sizes < 1 || cfg->num_sizes > 8)
      return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: need 1..8 progressive sizes");
    for (int i = 0; i < cfg->num_sizes; ++i)
      if (cfg->sizes[i] <= 0) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: sizes must be > 0");
  }
  if ((cfg->rule == CPA_RULE_PREDICTOR || cfg->rule == CPA_RULE_CALIBRATED) &&
      (cfg->pred.align <= 0 || cfg->pred.base_chunk_size <= 0))
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: predictor config needs align, base > 0");
  cpa_sched_s* s = new (std::nothrow) cpa_sched_s;
  if (!s) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_create: out of host memory");
  s->cfg = *cfg;
  *out = s;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_destroy(cpa_sched s) {
  delete s;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_add(cpa_sched s, int32_t prompt_len, int32_t max_new,
                                    int32_t arrival_step, int32_t* request_id) {
  if (!s) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_add: null scheduler");
  if (prompt_len <= 0 || max_new < 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_add: need prompt_len > 0, max_new >= 0");
  Req r;
  r.prompt_len = prompt_len;
  r.max_new = max_new;
  r.arrival = arrival_step;
  s->reqs.push_back(r);
  if (request_id) *request_id = (int32_t)s->reqs.size() - 1;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_set_model(cpa_sched s, double a, double b, double c, double T) {
  if (!s) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_set_model: null scheduler");
  s->cfg.a = a;
  s->cfg.b = b;
  s->cfg.c = c;
  s->cfg.T = T;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_form(cpa_sched s, int32_t capacity, int32_t* request_ids,
                                     int32_t* query_lens, int32_t* seq_lens, int32_t* num_seqs) {
  if (!s || !num_seqs || capacity < 0 || (capacity > 0 && (!request_ids || !query_lens || !seq_lens)))
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_form: bad arguments");
  if (s->formed) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_form: commit the formed batch first");
  std::vector<Entry> batch;
  int64_t left = s->cfg.budget;
  std::vector<int32_t> live;
  for (int32_t id : s->admitted)
    if (!s->reqs[id].done()) live.push_back(id);
  for (int32_t id : live) {  // decode rows
    const Req& r = s->reqs[id];
    if (r.prefilled == r.prompt_len && left > 0) {
      batch.push_back({id, 1, r.prompt_len + r.generated + 1});
      left -= 1;
    }
  }
  bool ran_out = false;
  for (int32_t id : live) {  // unfinished prefills
    const Req& r = s->reqs[id];
    if (r.prefilled >= r.prompt_len) continue;
    if (left <= 0) {
      ran_out = true;
      break;
    }
    const int32_t rem = r.prompt_len - r.prefilled;
    int64_t cap;
    const cpa_status st = cap_of(s, r.prefilled, rem, r.chunks, &cap);
    if (st != CPA_OK) return st;
    const int64_t chunk = std::min<int64_t>({(int64_t)rem, left, cap});
    if (chunk > 0) {
      batch.push_back({id, (int32_t)chunk, r.prefilled + (int32_t)chunk});
      left -= chunk;
    }
  }
  std::vector<int32_t> newly;
  if (!ran_out) {  // new requests, by arrival (ties by insertion)
    std::vector<int32_t> waiting;
    for (int32_t id = 0; id < (int32_t)s->reqs.size(); ++id)
      if (!s->reqs[id].admitted && s->reqs[id].arrival <= s->step) waiting.push_back(id);
    std::stable_sort(waiting.begin(), waiting.end(), [&](int32_t x, int32_t y) {
      return s->reqs[x].arrival < s->reqs[y].arrival;
    });
    for (int32_t id : waiting) {
      if (left <= 0) break;
      const Req& r = s->reqs[id];
      int64_t cap;
      const cpa_status st = cap_of(s, 0, r.prompt_len, 0, &cap);
      if (st != CPA_OK) return st;
      const int64_t chunk = std::min<int64_t>({(int64_t)r.prompt_len, left, cap});
      if (chunk <= 0) break;
      newly.push_back(id);
      batch.push_back({id, (int32_t)chunk, (int32_t)chunk});
      left -= chunk;
    }
  }
  if ((int32_t)batch.size() > capacity) {
    *num_seqs = (int32_t)batch.size();
    return cpa::fail(CPA_ERR_INVALID_ARG, "sched_form: capacity " + std::to_string(capacity) +
                                              " < " + std::to_string(batch.size()) + " sequences");
  }
  for (int32_t id : newly) {
    s->reqs[id].admitted = true;
    s->admitted.push_back(id);
  }
  for (size_t i = 0; i < batch.size(); ++i) {
    request_ids[i] = batch[i].rid;
    query_lens[i] = batch[i].q;
    seq_lens[i] = batch[i].n;
  }
  *num_seqs = (int32_t)batch.size();
  s->pending = batch;
  s->formed = true;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_commit(cpa_sched s) {
  if (!s) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_commit: null scheduler");
  if (!s->formed) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_commit: no formed batch");
  for (const Entry& e : s->pending) {
    Req& r = s->reqs[e.rid];
    if (r.prefilled == r.prompt_len) {
      r.generated += 1;
    } else {
      r.prefilled += e.q;
      r.chunks += 1;
    }
  }
  s->pending.clear();
  s->formed = false;
  s->step += 1;
  return cpa::ok();
}

extern "C" cpa_status cpa_sched_status(cpa_sched s, int32_t* finished, int32_t* step) {
  if (!s) return cpa::fail(CPA_ERR_INVALID_ARG, "sched_status: null scheduler");
  bool all = true;
  for (const Req& r : s->reqs) all = all && r.done();
  if (finished) *finished = all ? 1 : 0;
  if (step) *step = s->step;
  return cpa::ok();
}
