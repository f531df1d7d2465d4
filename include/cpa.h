/*
 * cpa.h -- C ABI of libcpa: paged chunked-prefill attention on gfx950.
 *
 * The library computes, on one AMD Instinct MI355X (gfx950), the attention
 * step of chunked prefill: a chunk of C new query tokens of a sequence
 * attends causally to the H tokens already in its paged KV cache plus
 * itself; decode rows (one query token) share the same call. It also holds
 * the host-side chunk-size predictor that sizes those chunks.
 *
 * Sources (cited by page title and section):
 *   [CPP]  vllm-ascend design document "Dynamic chunked pipeline parallel
 *          (CPP)": quadratic latency model, startup profiling, runtime
 *          prediction (solve f(L+x)-f(L)=T, smooth, align, cap), online
 *          calibration.
 *   [CP]   "vLLM Chunked-Prefills" article: section 3.1 (chunks cache their
 *          KV; token budget), section 3.2.1 (chunked attention over
 *          concatenated cached + new K/V), section 2.2.3 (a flattened
 *          token axis for batched tokens).
 *   [DS]   Ascend "dual-stream parallel for Qwen3 dense" article,
 *          section 3.1: attn_metadata fields num_actual_tokens,
 *          slot_mapping [bs], seq_lens [batch] (prefix + current tokens),
 *          query_lens [batch], block_table [batch, num_blocks].
 *
 * Conventions for every entry point:
 *   - Return a cpa_status; CPA_OK is 0, errors are negative. On error,
 *     cpa_last_error() returns a message for the calling thread. No C++
 *     exception crosses this boundary.
 *   - Device pointers are owned by the caller, must stay valid until the
 *     work queued on `stream` has finished, and are never freed here. The
 *     library allocates no device memory; host memory it allocates belongs
 *     to a plan and is released by cpa_plan_destroy.
 *   - GPU work is queued on `stream` (a hipStream_t; 0 = the null stream)
 *     and is asynchronous to the host. Host arrays are read during the call
 *     only.
 *   - bf16 tensors are raw 16-bit bfloat16 bit patterns, row-major,
 *     contiguous, 16-byte aligned.
 *   - Contents of device index arrays (slot_mapping, block_table) are
 *     trusted for speed, and the kernels never touch memory outside the
 *     cache for them: a slot outside [0, num_blocks * page_size) is not
 *     written, and a key whose block-table entry lies outside
 *     [0, num_blocks) reads as zero K and V rows (score 0, so it still takes
 *     part in the softmax). cpa_validate_metadata checks them on the host.
 */
#ifndef CPA_H_
#define CPA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cpa_status;
#define CPA_OK 0
#define CPA_ERR_INVALID_ARG (-1) /* bad pointer, size, or metadata */
#define CPA_ERR_UNSUPPORTED (-2) /* valid but not implemented (e.g. head_dim) */
#define CPA_ERR_WORKSPACE (-3)   /* workspace too small, or holds another plan */
#define CPA_ERR_HIP (-4)         /* a HIP runtime call or launch failed */
#define CPA_ERR_NUMERIC (-5)     /* non-finite or degenerate numeric input */

#define CPA_DTYPE_BF16 0
#define CPA_DTYPE_F32 1

/* Message for the last failed call on this thread ("" if none). */
const char* cpa_last_error(void);
/* Library version string. */
const char* cpa_version(void);

/*
 * One attention layer's shape.
 *   num_q_heads, num_kv_heads: Hq and Hkv, Hq % Hkv == 0; query head h
 *     reads KV head h / (Hq/Hkv) (contiguous groups).
 *   head_dim: d, 64 or 128.
 *   page_size: P tokens per cache page, a power of two, 16..1024.
 *   num_blocks: NB physical pages in each cache buffer.
 *   max_blocks_per_seq: row stride of block_table.
 *   scale: softmax scale applied to Q.K (normally 1/sqrt(d)).
 *   out_dtype: CPA_DTYPE_BF16 or CPA_DTYPE_F32 for the attention output.
 * Cache layout ([DS] section 3.1 leaves it open): K and V are separate
 * buffers of [NB, Hkv, P, d] bf16; slot s is page s / P, offset s % P.
 */
typedef struct cpa_layer_desc {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  float scale;
  int32_t out_dtype;
} cpa_layer_desc;

/*
 * KV write ([DS] section 3.1, slot_mapping; [CP] section 3.1, each chunk
 * caches its KV). For every token t < num_tokens with slot_mapping[t] >= 0:
 *   k_cache[slot/P, h, slot%P, :] = k_new[t, h, :]   for h < Hkv
 * and the same for v. Slots < 0 are skipped (padding); slots >= NB*P are
 * skipped. Duplicate slots within one call give an unspecified winner.
 *   k_new, v_new: device [num_tokens, Hkv, d] bf16.
 *   slot_mapping: device [num_tokens] int32.
 *   k_cache, v_cache: device [NB, Hkv, P, d] bf16, written in place.
 * num_tokens == 0 queues nothing and returns CPA_OK.
 */
cpa_status cpa_kv_write(const cpa_layer_desc* desc, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping,
                        int32_t num_tokens, void* k_cache, void* v_cache,
                        hipStream_t stream);

/*
 * Attention plan. Built on the host from host copies of query_lens and
 * seq_lens ([DS] section 3.1); it splits the flattened batch into work
 * items (sequence, KV head, query tile, key range) and sizes the device
 * workspace. A plan is immutable and may serve any number of layers that
 * share the same metadata (same desc shape and lengths).
 */
typedef struct cpa_plan_s* cpa_plan;

/* Tuning knobs; zero selects the default for a field. */
typedef struct cpa_plan_options {
  int32_t target_items;     /* work items to aim for (default: one per CU) */
  int32_t num_cus;          /* compute units to plan for (default 256) */
  int32_t prefill_split;    /* force this many key splits per prefill
                               tile (default: chosen from the work) */
  int32_t decode_split_keys;/* keys per decode split (default: the largest
                               of 2048, 1024, 512 that still gives 4 decode
                               items per CU, else 256) */
  int32_t min_split_keys;   /* smallest prefill split piece in keys, a
                               multiple of 64; nonzero also keeps splits
                               that the planner's cost rule would drop
                               (default 0: chosen from the work) */
} cpa_plan_options;

/*
 * Builds a plan for num_seqs sequences. Sequence s contributes
 * query_lens[s] tokens to the flat token axis (in order s = 0, 1, ...) at
 * absolute positions seq_lens[s]-query_lens[s] .. seq_lens[s]-1; it sees
 * its prefix of H = seq_lens[s]-query_lens[s] cached tokens plus itself,
 * causally. Rows with query_len == 1 are decode rows; others are prefill
 * chunks; query_len == 0 contributes nothing.
 * Validates: 0 <= query_len <= seq_len, ceil(seq_len/P) <=
 * max_blocks_per_seq, head_dim in {64, 128}, Hq % Hkv == 0, page_size a
 * power of two in 16..1024, total tokens < 2^31.
 *   options may be NULL. *workspace_bytes receives the device workspace
 *   size cpa_attention needs. On error *out_plan is NULL.
 * A plan of more than 2^21 work items or 2^31 - 1 split-partial rows (tiny
 * decode_split_keys over long rows, huge prefill_split) is refused with
 * CPA_ERR_UNSUPPORTED.
 */
cpa_status cpa_plan_create(const cpa_layer_desc* desc,
                           const int32_t* query_lens, const int32_t* seq_lens,
                           int32_t num_seqs, const cpa_plan_options* options,
                           cpa_plan* out_plan, size_t* workspace_bytes);

cpa_status cpa_plan_destroy(cpa_plan plan);

typedef struct cpa_plan_info {
  int32_t num_seqs;
  int32_t num_tokens;          /* sum of query_lens */
  int32_t num_prefill_items;   /* work items of the MFMA kernel */
  int32_t num_decode_items;    /* work items of the decode kernel */
  int32_t num_combine_items;   /* tiles whose key range was split */
  int32_t num_partial_rows;    /* split-partial rows in the workspace: O/l in the
                                  output's precision, fp32 max and sum */
  int64_t visible_pairs;       /* sum over rows and q heads of keys seen */
  size_t workspace_bytes;
} cpa_plan_info;

cpa_status cpa_plan_get_info(cpa_plan plan, cpa_plan_info* info);

/*
 * Copies the plan's work lists into `workspace` (device, at least
 * workspace_bytes as returned by cpa_plan_create, 256-byte aligned), queued
 * on `stream`. A workspace holds one plan at a time: uploading another plan
 * into the same workspace replaces it, and cpa_attention then refuses the
 * first plan with CPA_ERR_WORKSPACE. The copy reads the plan's host-side
 * image: keep the plan alive until `stream` has passed the upload.
 */
cpa_status cpa_plan_upload(cpa_plan plan, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked-prefill / decode attention over the plan's flattened batch
 * ([CP] section 3.2.1 with a causal mask offset by the prefix; [DS]
 * section 3.1 metadata). For every sequence s, query row i < query_len[s]
 * (flat token t = sum(query_lens[:s]) + i, absolute position p = H_s + i)
 * and query head h (KV head g = h / (Hq/Hkv)):
 *   out[t, h, :] = sum_{j <= p} softmax_j(scale * q[t,h,:].K_j) * V_j
 * where K_j = k_cache[block_table[s, j/P], g, j%P, :] and V_j likewise.
 * The chunk's own K/V must already be in the cache (cpa_kv_write).
 *   q: device [T, Hq, d] bf16.   k_cache, v_cache: device [NB, Hkv, P, d].
 *   block_table: device [num_seqs, max_blocks_per_seq] int32.
 *   out: device [T, Hq, d], bf16 or fp32 per desc->out_dtype.
 *   workspace: the buffer passed to cpa_plan_upload for this plan.
 * Arithmetic: bf16 MFMA products, fp32 accumulation and softmax. Rows
 * whose keys were split over several work items are merged by a later
 * kernel (one launch for split prefill tiles, one for split decode rows)
 * from partials kept in the output's precision (bf16 or fp32), with fp32
 * max and sum.
 */
cpa_status cpa_attention(cpa_plan plan, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         void* out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * One batch step's KV write and attention in one call: the results (out
 * and both caches) are those of cpa_kv_write(desc, k_new, v_new,
 * slot_mapping, T, k_cache, v_cache) followed by cpa_attention(plan, q,
 * k_cache, v_cache, block_table, ...), with T the plan's token count
 * ([DS] section 3.1: slot_mapping places every new token's K/V in the
 * cache; [CP] section 3.2.1: attention over cached and new keys).
 * Fusing the two is this library's own design; [DS] and [CP] run them as
 * two steps.
 * The prefill kernel writes the new rows itself and reads every key at a
 * position >= H_s of its sequence from k_new / v_new instead of the cache,
 * so the write and the reads need no ordering and the separate write
 * launch disappears; decode rows read the cache in a later kernel. The
 * equality therefore assumes consistent metadata: every new token's slot
 * is block_table[s, p/P]*P + p%P for its position p (cpa_validate_metadata
 * checks bounds, not this). Without prefill items, or when the step has
 * more new rows than its prefill threads take, the KV-write kernel runs
 * first and the attention follows as in cpa_attention.
 *   k_new, v_new: device [T, Hkv, d] bf16. slot_mapping: device [T] int32.
 *   Other arguments, layouts, ownership and errors as cpa_kv_write and
 *   cpa_attention; a NULL pointer gives CPA_ERR_INVALID_ARG.
 */
cpa_status cpa_kv_write_attention(cpa_plan plan, const void* q, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping,
                                  void* k_cache, void* v_cache,
                                  const int32_t* block_table, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * call and results as cpa_kv_write_attention, with no workspace argument:
 * the plan's work lists and split partials live in a static device array of
 * CPA_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends. The call allocates nothing; when the
 * array on the current device does not hold this plan's work lists (the
 * first call, or another plan's call came in between) it uploads them there
 * first, as cpa_plan_upload does (an asynchronous host-to-device copy on
 * `stream` from the plan's host image: keep the plan alive until `stream`
 * has passed it).
 *   Limit: a plan whose workspace_bytes exceeds CPA_STATIC_SCRATCH_BYTES is
 *   refused with CPA_ERR_WORKSPACE before any GPU work.
 *   Sharing: every call on one GPU uses that GPU's one array. Calls that
 *   overlap on one GPU (other streams, other host threads, other plans)
 *   race on it; the caller orders them. cpa_plan_upload / cpa_attention on
 *   caller workspaces are unaffected.
 *   Other arguments, layouts, ownership and errors as cpa_kv_write_attention.
 */
#define CPA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
cpa_status cpa_kv_write_attention_static(cpa_plan plan, const void* q, const void* k_new,
                                         const void* v_new, const int32_t* slot_mapping,
                                         void* k_cache, void* v_cache,
                                         const int32_t* block_table, void* out,
                                         hipStream_t stream);

/*
 * Host-side bounds check of metadata before it is trusted on the device:
 * every slot_mapping entry is < 0 or < NB*P and no slot repeats; every
 * block_table entry a sequence can reach (j < ceil(seq_len/P)) is in
 * [0, NB); lengths as in cpa_plan_create. Any pointer may be NULL to skip
 * that check. Returns CPA_ERR_INVALID_ARG naming the first bad entry.
 */
cpa_status cpa_validate_metadata(const cpa_layer_desc* desc,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 const int32_t* block_table,
                                 const int32_t* query_lens,
                                 const int32_t* seq_lens, int32_t num_seqs);

/* ---- Chunk-size predictor ([CPP]; pure host fp64, no GPU needed) ---- */

/*
 * base_chunk_size: the base chunk (the profile's largest size).
 * align: alignment quantum ([CPP] "runtime": a page-size multiple).
 * min_chunk: floor after alignment ([CPP]: at least 64).
 * max_chunk: cap ([CPP]: max_num_scheduled_tokens).
 * max_model_len: cap on L + chunk ([CPP]: max_model_len - history_len).
 * smooth_factor: s in xs = s*x + (1-s)*base ([CPP] "runtime" names the
 *   blend but prints no formula; this linear blend is the reading taken).
 */
typedef struct cpa_predictor_cfg {
  int64_t base_chunk_size;
  int64_t align;
  int64_t min_chunk;
  int64_t max_chunk;
  int64_t max_model_len;
  double smooth_factor;
} cpa_predictor_cfg;

/*
 * [CPP] "startup: profiling": n distinct sizes spread evenly from base down
 * to lo: sizes[i] = round(base - i*(base-lo)/(n-1)) (round half to even).
 * Needs n >= 2, base > lo >= 1 and base - lo >= n - 1 (else the sizes could
 * not all differ): CPA_ERR_INVALID_ARG otherwise.
 */
cpa_status cpa_predictor_profile_sizes(int64_t base, int32_t n, int64_t lo,
                                       int64_t* sizes);

/*
 * [CPP] "quadratic latency model" + "startup": least-squares fit of
 * ms ~ a*l^2 + b*l + c over n >= 3 points (fp64, columns scaled by the
 * largest |l|). CPA_ERR_NUMERIC if the points are non-finite or do not
 * determine three coefficients.
 */
cpa_status cpa_predictor_fit(const double* lens, const double* ms, int32_t n,
                             double* a, double* b, double* c);

/* [CPP] "runtime": T = f(base) - f(0) = a*base^2 + b*base. */
cpa_status cpa_predictor_target(const cpa_predictor_cfg* cfg, double a,
                                double b, double* T);

/*
 * [CPP] "runtime": chunk size for the next chunk at prefix history_len with
 * `remaining` prompt tokens left. x is the positive root of
 * a*x^2 + (2aL+b)*x - T = 0 (quadratic formula); if a <= 0 or a value is
 * non-finite, x = T/b when b > 0, else base. Then xs = s*x + (1-s)*base,
 * xi = floor(xs + 1e-6), aligned down to `align`, raised to min_chunk and
 * capped at max_chunk, max_model_len - history_len and remaining (never
 * below 0). *raw_x (may be NULL) receives x.
 */
cpa_status cpa_predictor_next_chunk(const cpa_predictor_cfg* cfg, double a,
                                    double b, double T, int64_t history_len,
                                    int64_t remaining, int64_t* chunk,
                                    double* raw_x);

/* ---- Two-micro-batch split ([DS] section 3.1; host) ---- */

enum { CPA_SPLIT_SIMPLE = 0, CPA_SPLIT_BALANCED = 1 };

/*
 * Split point of a flattened batch into two micro-batches ([DS] section
 * 3.1 "data split"). CPA_SPLIT_SIMPLE: seq_split = num_seqs / 2.
 * CPA_SPLIT_BALANCED: the boundary k in 1 .. num_seqs-1 whose running token
 * count sum(query_lens[:k]) is nearest total/2 (ties to the smaller k); the
 * split is refused when |n1 - n2| / min(n1, n2) > balance_threshold, or
 * either micro-batch has fewer than length_threshold tokens, or one of them
 * is empty. token_split = sum(query_lens[:seq_split]). A refused split (or
 * num_seqs < 2) returns CPA_OK with *seq_split = *token_split = 0.
 *
 * The micro-batches are then: sequences [0, seq_split) and [seq_split,
 * num_seqs) (query_lens, seq_lens, block_table rows), tokens [0,
 * token_split) and [token_split, num_tokens) (q, out, k_new, v_new,
 * slot_mapping rows). Each half is planned with cpa_plan_create on its own
 * lengths and run with cpa_attention on pointers offset by those rows, in
 * its own workspace; halves on two streams may run concurrently.
 */
cpa_status cpa_split_point(const int32_t* query_lens, int32_t num_seqs, int32_t mode,
                           double balance_threshold, int32_t length_threshold,
                           int32_t* seq_split, int32_t* token_split);

/* ---- Online calibration ([CPP] "online calibration"; host fp64) ---- */

/*
 * Two-variable latency model f(C, H) = a*C*(C+H) + b*(C+H) + c of a chunk of
 * C tokens after H tokens of history. An executed batch is recorded by its
 * feature vector feat = [sum C*(C+H), sum (C+H), N] over its N sequences
 * with C > 0 ([CPP] prints this vector), so batch time ~ a*feat[0] +
 * b*feat[1] + c*feat[2]. chunk_lens/hist_lens: host arrays of n entries
 * (read during the call); hist_lens >= 0. feat: 3 doubles written.
 */
cpa_status cpa_calib_features(const int32_t* chunk_lens, const int32_t* hist_lens,
                              int32_t n, double* feat);

/*
 * Least squares (a, b, c) over n >= 3 records: feats is row-major [n][3],
 * ms the measured times (any unit; the coefficients take it). Columns are
 * scaled by their largest magnitude before the solve. CPA_ERR_NUMERIC for
 * non-finite input, an all-zero column, or records that do not determine
 * three coefficients.
 */
cpa_status cpa_calib_fit(const double* feats, const double* ms, int32_t n,
                         double* a, double* b, double* c);

/*
 * Per-chunk target of the two-variable model: T' = f(base, 0) =
 * a*base^2 + b*base + c (the latency of a base-size chunk without history;
 * [CPP] leaves the target of the calibrated model unstated, this is the
 * reading taken).
 */
cpa_status cpa_calib_target(const cpa_predictor_cfg* cfg, double a, double b,
                            double c, double* T);

/*
 * Next chunk at prefix history_len under the two-variable model: x is the
 * positive root of a*x^2 + (a*H + b)*x + (b*H + c - T) = 0 (f(x, H) = T,
 * quadratic formula); if a <= 0 (all values finite) x = (T - b*H - c) /
 * (a*H + b) when a*H + b > 0, else base; a negative discriminant or a
 * non-finite value gives base. Then the post-processing of
 * cpa_predictor_next_chunk (smoothing, floor(xs + 1e-6), alignment,
 * min_chunk, caps). *raw_x (may be NULL) receives x.
 */
cpa_status cpa_calib_next_chunk(const cpa_predictor_cfg* cfg, double a,
                                double b, double c, double T,
                                int64_t history_len, int64_t remaining,
                                int64_t* chunk, double* raw_x);

/*
 * Record window of the online calibration ([CPP]: refit by least squares
 * once enough points, 5 to 30, are held): the `window` most recent records
 * are kept, and the model is refitted after every record once at least
 * min_points are held (3 <= min_points <= window). Host object owned by the
 * caller; not thread-safe.
 */
typedef struct cpa_calib_s* cpa_calib;
cpa_status cpa_calib_create(int32_t min_points, int32_t window, cpa_calib* out);
cpa_status cpa_calib_destroy(cpa_calib calib);

/*
 * Adds one record (feat: 3 doubles as from cpa_calib_features; ms its
 * time). *ready (may be NULL) is set to 1 once a model is available. A
 * failed refit (CPA_ERR_NUMERIC) keeps the previous model.
 */
cpa_status cpa_calib_record(cpa_calib calib, const double* feat, double ms,
                            int32_t* ready);

/*
 * Current model. *points (may be NULL) receives the records held.
 * CPA_ERR_NUMERIC while fewer than min_points records have been fitted.
 */
cpa_status cpa_calib_model(cpa_calib calib, double* a, double* b, double* c,
                           int32_t* points);

/* ---- Token-budget batch former ([CP] section 3.1; host) ---- */

enum {
  CPA_RULE_FIXED = 0,        /* chunk cap = fixed_chunk ([CP] 3.1: typically 512) */
  CPA_RULE_PROGRESSIVE = 1,  /* k-th chunk of a request capped by sizes[min(k, n-1)] ([CP] 3.2.2) */
  CPA_RULE_PREDICTOR = 2,    /* cpa_predictor_next_chunk(pred, a, b, T, L, remaining) ([CPP]) */
  CPA_RULE_CALIBRATED = 3    /* cpa_calib_next_chunk(pred, a, b, c, T, L, remaining) ([CPP]) */
};

typedef struct cpa_sched_cfg {
  int32_t budget;           /* tokens per step (> 0) */
  int32_t rule;             /* CPA_RULE_* */
  int32_t fixed_chunk;      /* CPA_RULE_FIXED */
  int32_t num_sizes;        /* CPA_RULE_PROGRESSIVE: 1..8 */
  int32_t sizes[8];
  cpa_predictor_cfg pred;   /* predictor / calibrated rules */
  double a, b, c, T;        /* model coefficients and target of those rules */
} cpa_sched_cfg;

typedef struct cpa_sched_s* cpa_sched;
cpa_status cpa_sched_create(const cpa_sched_cfg* cfg, cpa_sched* out);
cpa_status cpa_sched_destroy(cpa_sched sched);

/* A request of prompt_len > 0 tokens generating max_new >= 0 tokens after
 * its prompt, admissible from step arrival_step on. Ids count from 0. */
cpa_status cpa_sched_add(cpa_sched sched, int32_t prompt_len, int32_t max_new,
                         int32_t arrival_step, int32_t* request_id);

/* New model coefficients for the predictor / calibrated rules (e.g. from
 * cpa_calib_model and cpa_calib_target); used from the next formed batch. */
cpa_status cpa_sched_set_model(cpa_sched sched, double a, double b, double c, double T);

/*
 * Forms the current step's batch within the budget ([CP] 3.1): first one
 * decode row per admitted request whose prompt is prefilled (query_len 1,
 * seq_len = prompt_len + generated + 1), then one chunk per unfinished
 * prefill, chunk = min(remaining prompt, budget left, rule cap at prefix L),
 * then, if the unfinished prefills did not exhaust the budget, new requests
 * in arrival order (ties by id) while budget is left. Decode rows and
 * unfinished prefills are visited in admission order. A request whose
 * prompt completes becomes a decode row from the next step; it finishes
 * after max_new decode rows. Writes up to `capacity` entries (request id,
 * query_len, seq_len, in flattened-axis order) and *num_seqs;
 * CPA_ERR_INVALID_ARG (state unchanged, *num_seqs = the size needed) when
 * capacity is too small. Call cpa_sched_commit after running the batch.
 */
cpa_status cpa_sched_form(cpa_sched sched, int32_t capacity, int32_t* request_ids,
                          int32_t* query_lens, int32_t* seq_lens, int32_t* num_seqs);

/* Advances the requests by the formed batch and the step counter. */
cpa_status cpa_sched_commit(cpa_sched sched);

/* *finished = 1 once every request is done; *step = steps committed. */
cpa_status cpa_sched_status(cpa_sched sched, int32_t* finished, int32_t* step);

#ifdef __cplusplus
}
#endif

#endif /* CPA_H_ */
