// C ABI entry points of libcpa, and the host-side attention planner.
//
// The planner turns the per-sequence metadata of a flattened batch (the
// Ascend dual-stream article, section 3.1: query_lens and seq_lens per
// sequence, tokens concatenated on one axis, seq_len = prefix + current)
// into lists of work items for the kernels:
//   * prefill chunks (query_len >= 2): one item per (sequence, KV head,
//     head sub-group, 256-row query tile), the key range split into pieces
//     when there are too few tiles to fill the GPU; split tiles also get a
//     combine item;
//   * decode rows (query_len == 1): one item per (sequence, KV head, key
//     range of decode_split_keys), merged by a combine item when split.
// Items are then ordered for the XCDs (order_for_xcds): each (sequence,
// KV head) group on one XCD, the groups balanced over the XCDs, the
// costliest items of an XCD first.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "cpa.h"
#include "cpa_host.h"
#include "cpa_internal.h"

namespace cpa {

std::string& last_error() {
  thread_local std::string msg;
  return msg;
}

namespace {

constexpr size_t kAlign = 256;
constexpr int kDefaultCus = 256;
constexpr int kNumXcds = 8;
// A split costs the combine launch that merges its pieces, measured at
// about as much as two 64-key tiles of one item (at d = 64 and d = 128
// alike: a lone item's tiles are bound by memory latency, not by the
// products): a tile is split only when that shortens the longest item by
// more. In the d = 64 kernel, an item of at most 64 packed rows has six
// of its eight waves idle (they skip their phases), so its tiles cost about
// half as much and the split must save twice as many of them: measured,
// 4-tile items of 32-64 rows ran 0.25-0.35 us faster unsplit, 5-tile items
// tied, and items of 96-128 rows or of 6+ tiles still gained from the split.
constexpr int kCombineTiles = 2;
constexpr int kSmallItemRows = 64;
// Default keys per decode split: the largest of these that still gives
// every CU kDecodeItemsPerCu decode items, else the smallest. Longer
// splits mean fewer item starts and merges (the LLaMA-13B decode rows run
// 1.5% faster at 2048 than at 512 keys), shorter ones fill the GPU when
// the decode rows are few.
constexpr int kDecodeSplitChoices[] = {2048, 1024, 512, 256};
constexpr int kDecodeItemsPerCu = 4;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

cpa_status hip_fail(hipError_t e, const char* what) {
  return fail(CPA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return ((1 << l) == v) ? l : -1;
}

cpa_status check_desc(const cpa_layer_desc* d) {
  if (!d) return fail(CPA_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
    return fail(CPA_ERR_INVALID_ARG, "need num_q_heads > 0, num_kv_heads > 0, Hq % Hkv == 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(CPA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int pl = log2_exact(d->page_size);
  if (d->page_size < 16 || d->page_size > 1024 || pl < 0)
    return fail(CPA_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 1024]");
  if (d->num_blocks <= 0 || d->max_blocks_per_seq <= 0)
    return fail(CPA_ERR_INVALID_ARG, "num_blocks and max_blocks_per_seq must be > 0");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale))
    return fail(CPA_ERR_NUMERIC, "scale must be finite and > 0");
  if (d->out_dtype != CPA_DTYPE_BF16 && d->out_dtype != CPA_DTYPE_F32)
    return fail(CPA_ERR_INVALID_ARG, "out_dtype must be CPA_DTYPE_BF16 or CPA_DTYPE_F32");
  if ((int64_t)d->num_blocks * d->page_size >= (int64_t)1 << 31)
    return fail(CPA_ERR_UNSUPPORTED, "num_blocks * page_size must be < 2^31 slots");
  return CPA_OK;
}

cpa_status check_lens(const cpa_layer_desc* d, const int32_t* ql, const int32_t* sl, int32_t S,
                      int64_t* total_tokens) {
  if (S < 0) return fail(CPA_ERR_INVALID_ARG, "num_seqs < 0");
  if (S > 0 && (!ql || !sl)) return fail(CPA_ERR_INVALID_ARG, "query_lens/seq_lens is NULL");
  int64_t total = 0;
  for (int32_t s = 0; s < S; ++s) {
    if (ql[s] < 0 || ql[s] > sl[s])
      return fail(CPA_ERR_INVALID_ARG, "sequence " + std::to_string(s) +
                                           ": need 0 <= query_len <= seq_len");
    const int64_t pages = ((int64_t)sl[s] + d->page_size - 1) / d->page_size;
    if (pages > d->max_blocks_per_seq)
      return fail(CPA_ERR_INVALID_ARG, "sequence " + std::to_string(s) +
                                           ": ceil(seq_len/page_size) > max_blocks_per_seq");
    total += ql[s];
  }
  if (total >= ((int64_t)1 << 31) / std::max(1, d->num_q_heads))
    return fail(CPA_ERR_UNSUPPORTED, "too many tokens for 32-bit row indices");
  *total_tokens = total;
  return CPA_OK;
}

// Which plan currently owns which workspace.
std::mutex g_ws_mu;
std::unordered_map<const void*, uint64_t> g_ws_owner;
uint64_t g_next_plan_id = 1;

}  // namespace
}  // namespace cpa

struct cpa_plan_s {
  cpa_layer_desc desc;
  int32_t num_seqs = 0, num_tokens = 0;
  int32_t group = 1;             // Hq / Hkv
  int32_t decode_group = 0;      // heads per decode item, 0 if no decode kernel
  int32_t part_rows = 0;
  // Combine items of split prefill tiles come first, then those of split
  // decode rows; each group has its own launch, sized by its own largest
  // row count and split count (a decode tile has G rows, a prefill tile up
  // to 256, and one grid for both would be mostly empty blocks).
  int32_t combine_count[2] = {0, 0}, combine_rows[2] = {0, 0}, combine_splits[2] = {0, 0};
  int32_t part_bf16 = 0;         // split partials O/l in bf16 (else fp32)
  int32_t prefill_max_rows = 0;  // largest nq * nheads of a prefill item
  int64_t visible_pairs = 0;
  std::vector<cpa::WorkItem> prefill, decode;
  std::vector<cpa::CombineItem> combine;
  size_t off_prefill = 0, off_decode = 0, off_combine = 0, off_part_o = 0, off_part_ml = 0;
  size_t ws_bytes = 0;
  uint64_t id = 0;
  std::vector<uint8_t> image;    // host copy of the work lists, uploaded as is
};

namespace {

struct Tile {
  int32_t seq, kvh, head0, nheads, tok0, q0, nq, hist, kv_len;
};

// Largest plan: work items (48 bytes each, on the host and in the
// workspace) and partial rows (indexed in 32 bits by the kernels).
constexpr int64_t kMaxPlanItems = (int64_t)1 << 21;
constexpr int64_t kMaxPartialRows = ((int64_t)1 << 31) - 1;

// Appends the items of tile t; false (nothing appended) if the plan would
// outgrow kMaxPlanItems or kMaxPartialRows.
bool add_split(cpa_plan_s* p, std::vector<cpa::WorkItem>& out, const Tile& t, int64_t nsplit,
               int align) {
  cpa::WorkItem base{t.seq, t.kvh, t.head0, t.nheads, t.tok0, t.q0, t.nq, t.hist, 0, t.kv_len, -1, 0};
  // The key range is cut into `align`-key units dealt out as evenly as
  // possible (piece sizes differ by at most one unit), so split items of a
  // tile finish together.
  const int64_t units = ((int64_t)t.kv_len + align - 1) / align;
  nsplit = std::min(nsplit, units);
  const int64_t items = (int64_t)p->prefill.size() + (int64_t)p->decode.size();
  if (items + std::max<int64_t>(nsplit, 1) > kMaxPlanItems) return false;
  if (nsplit <= 1) {
    out.push_back(base);
    return true;
  }
  const int rows = t.nq * t.nheads;
  if ((int64_t)p->part_rows + nsplit * rows > kMaxPartialRows) return false;
  const int part0 = p->part_rows;
  p->part_rows += (int)(nsplit * rows);
  const int grp = (&out == &p->decode) ? 1 : 0;
  p->combine_count[grp] += 1;
  p->combine_rows[grp] = std::max(p->combine_rows[grp], rows);
  p->combine_splits[grp] = std::max(p->combine_splits[grp], (int)nsplit);
  p->combine.push_back(
      cpa::CombineItem{t.tok0, t.head0, t.nheads, t.nq, (int)nsplit, part0, rows, 0});
  int64_t start = 0;
  for (int64_t k = 0; k < nsplit; ++k) {
    const int64_t n_units = units / nsplit + (k < units % nsplit ? 1 : 0);
    cpa::WorkItem w = base;
    w.kv0 = (int32_t)(start * align);
    w.kv1 = (int32_t)std::min<int64_t>(t.kv_len, (start + n_units) * align);
    w.part = (int32_t)(part0 + k * rows);
    out.push_back(w);
    start += n_units;
  }
  return true;
}

int64_t item_cost(const cpa::WorkItem& w) {
  return (int64_t)(w.kv1 - w.kv0) * std::max(1, w.nq * w.nheads);
}

// Order work items for the hardware dispatcher, which hands workgroup i to
// XCD i % 8: items that read the same KV head of the same sequence are kept
// on one XCD (one L2), affinity groups are spread over the XCDs longest
// first, and inside an XCD the costliest items go first.
void order_for_xcds(std::vector<cpa::WorkItem>& v, int nxcd) {
  if (v.size() <= 1) return;
  std::vector<std::pair<int64_t, std::vector<cpa::WorkItem>>> groups;
  std::unordered_map<int64_t, size_t> index;
  for (const cpa::WorkItem& w : v) {
    const int64_t key = ((int64_t)w.seq << 32) | (uint32_t)w.kvh;
    auto it = index.find(key);
    if (it == index.end()) {
      it = index.emplace(key, groups.size()).first;
      groups.push_back({0, {}});
    }
    groups[it->second].first += item_cost(w);
    groups[it->second].second.push_back(w);
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const auto& x, const auto& y) { return x.first > y.first; });
  std::vector<std::vector<cpa::WorkItem>> bins(nxcd);
  std::vector<int64_t> load(nxcd, 0);
  for (auto& g : groups) {
    const int b = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[b] += g.first;
    bins[b].insert(bins[b].end(), g.second.begin(), g.second.end());
  }
  for (auto& b : bins) {
    std::stable_sort(b.begin(), b.end(), [](const cpa::WorkItem& x, const cpa::WorkItem& y) {
      return item_cost(x) > item_cost(y);
    });
    std::reverse(b.begin(), b.end());  // pop from the back = costliest first
  }
  std::vector<cpa::WorkItem> out;
  out.reserve(v.size());
  while (out.size() < v.size()) {
    const int x = (int)(out.size() % nxcd);
    int b = x;
    if (bins[b].empty()) {
      b = 0;
      for (int k = 1; k < nxcd; ++k)
        if (bins[k].size() > bins[b].size()) b = k;
    }
    out.push_back(bins[b].back());
    bins[b].pop_back();
  }
  v.swap(out);
}

}  // namespace

namespace {

// The step's new K/V rows for the fused entry point.
struct NewRows {
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
};

cpa_status attention_impl(cpa_plan plan, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, const NewRows* nr) {
  if (!plan) return cpa::fail(CPA_ERR_INVALID_ARG, "attention: plan is NULL");
  if (plan->num_tokens == 0) return cpa::ok();
  if (!q || !k_cache || !v_cache || !block_table || !out || !workspace)
    return cpa::fail(CPA_ERR_INVALID_ARG, "attention: NULL pointer");
  if (nr && (!nr->k_new || !nr->v_new || !nr->slot_mapping))
    return cpa::fail(CPA_ERR_INVALID_ARG, "kv_write_attention: NULL pointer");
  if (workspace_bytes < plan->ws_bytes)
    return cpa::fail(CPA_ERR_WORKSPACE, "attention: workspace smaller than the plan needs");
  {
    std::lock_guard<std::mutex> lk(cpa::g_ws_mu);
    auto it = cpa::g_ws_owner.find(workspace);
    if (it == cpa::g_ws_owner.end() || it->second != plan->id)
      return cpa::fail(CPA_ERR_WORKSPACE,
                       "attention: this plan was not uploaded to this workspace "
                       "(call cpa_plan_upload first)");
  }
  const cpa_layer_desc& d = plan->desc;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  cpa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.bt_stride = d.max_blocks_per_seq;
  a.num_q_heads = d.num_q_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.page_log2 = cpa::log2_exact(d.page_size);
  a.num_blocks = d.num_blocks;
  a.scale_log2e = d.scale * 1.4426950408889634f;
  a.out = out;
  a.out_f32 = d.out_dtype == CPA_DTYPE_F32;
  a.part_o = ws + plan->off_part_o;
  a.part_bf16 = plan->part_bf16;
  a.part_ml = reinterpret_cast<float*>(ws + plan->off_part_ml);
  a.zeros = reinterpret_cast<const uint16_t*>(ws);
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.slot_mapping = nullptr;
  a.k_cache_w = nullptr;
  a.v_cache_w = nullptr;
  a.num_new_tokens = 0;

  hipError_t e = hipSuccess;
  bool fused = false;
  if (nr) {
    // The prefill kernel takes the cache writes when its threads can hold
    // them (each writes at most kFusedWritesPerThread rows' chunks);
    // otherwise, or without prefill items, the KV-write kernel runs first.
    const int64_t chunks = (int64_t)plan->num_tokens * d.num_kv_heads * (d.head_dim / 8);
    const int64_t room = (int64_t)plan->prefill.size() * 64 * cpa::kPrefillWaves *
                         cpa::kFusedWritesPerThread;
    // (The kernel indexes the chunks in 32 bits.)
    fused = !plan->prefill.empty() && chunks <= room && room < ((int64_t)1 << 31);
    if (fused) {
      a.k_new = static_cast<const uint16_t*>(nr->k_new);
      a.v_new = static_cast<const uint16_t*>(nr->v_new);
      a.slot_mapping = nr->slot_mapping;
      a.k_cache_w = static_cast<uint16_t*>(nr->k_cache);
      a.v_cache_w = static_cast<uint16_t*>(nr->v_cache);
      a.num_new_tokens = plan->num_tokens;
    } else {
      e = cpa::launch_kv_write(static_cast<const uint16_t*>(nr->k_new),
                               static_cast<const uint16_t*>(nr->v_new), nr->slot_mapping,
                               plan->num_tokens, static_cast<uint16_t*>(nr->k_cache),
                               static_cast<uint16_t*>(nr->v_cache), d.num_kv_heads, d.head_dim,
                               a.page_log2, d.num_blocks, stream);
      if (e != hipSuccess) return cpa::hip_fail(e, "kv_write launch");
    }
  }
  e = cpa::launch_prefill(reinterpret_cast<const cpa::WorkItem*>(ws + plan->off_prefill),
                          (int)plan->prefill.size(), a, d.head_dim, fused,
                          plan->prefill_max_rows, stream);
  if (e != hipSuccess) return cpa::hip_fail(e, "prefill attention launch");
  e = cpa::launch_decode(reinterpret_cast<const cpa::WorkItem*>(ws + plan->off_decode),
                         (int)plan->decode.size(), a, d.head_dim, plan->decode_group, stream);
  if (e != hipSuccess) return cpa::hip_fail(e, "decode attention launch");
  const cpa::CombineItem* citems = reinterpret_cast<const cpa::CombineItem*>(ws + plan->off_combine);
  for (int g = 0; g < 2; ++g) {
    e = cpa::launch_combine(citems + (g ? plan->combine_count[0] : 0), plan->combine_count[g],
                            plan->combine_rows[g], plan->combine_splits[g], a, d.head_dim, stream);
    if (e != hipSuccess) return cpa::hip_fail(e, "split combine launch");
  }
  return cpa::ok();
}

}  // namespace

namespace cpa {

size_t plan_workspace_bytes(cpa_plan plan) { return plan ? plan->ws_bytes : 0; }

bool workspace_holds(cpa_plan plan, const void* workspace) {
  if (!plan) return false;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws_owner.find(workspace);
  return it != g_ws_owner.end() && it->second == plan->id;
}

}  // namespace cpa

extern "C" {

const char* cpa_last_error(void) { return cpa::last_error().c_str(); }

const char* cpa_version(void) { return "cpa 0.1.0 (gfx950)"; }

cpa_status cpa_kv_write(const cpa_layer_desc* desc, const void* k_new, const void* v_new,
                        const int32_t* slot_mapping, int32_t num_tokens, void* k_cache,
                        void* v_cache, hipStream_t stream) {
  cpa_status st = cpa::check_desc(desc);
  if (st != CPA_OK) return st;
  if (num_tokens < 0) return cpa::fail(CPA_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_tokens == 0) return cpa::ok();
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return cpa::fail(CPA_ERR_INVALID_ARG, "kv_write: NULL pointer");
  const hipError_t e = cpa::launch_kv_write(
      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping,
      num_tokens, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
      desc->num_kv_heads, desc->head_dim, cpa::log2_exact(desc->page_size), desc->num_blocks,
      stream);
  if (e != hipSuccess) return cpa::hip_fail(e, "kv_write launch");
  return cpa::ok();
}

cpa_status cpa_plan_create(const cpa_layer_desc* desc, const int32_t* query_lens,
                           const int32_t* seq_lens, int32_t num_seqs,
                           const cpa_plan_options* options, cpa_plan* out_plan,
                           size_t* workspace_bytes) {
  if (!out_plan || !workspace_bytes)
    return cpa::fail(CPA_ERR_INVALID_ARG, "plan_create: NULL output pointer");
  *out_plan = nullptr;
  cpa_status st = cpa::check_desc(desc);
  if (st != CPA_OK) return st;
  int64_t total = 0;
  st = cpa::check_lens(desc, query_lens, seq_lens, num_seqs, &total);
  if (st != CPA_OK) return st;
  cpa_plan_options opt{};
  if (options) opt = *options;
  if (opt.target_items < 0 || opt.num_cus < 0 || opt.prefill_split < 0 ||
      opt.decode_split_keys < 0 || opt.min_split_keys < 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "plan options must be >= 0");
  if (opt.min_split_keys % cpa::kSplitAlign != 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "min_split_keys must be a multiple of 64");

  cpa_plan_s* p = new (std::nothrow) cpa_plan_s();
  if (!p) return cpa::fail(CPA_ERR_INVALID_ARG, "plan_create: out of host memory");
  p->desc = *desc;
  p->num_seqs = num_seqs;
  p->num_tokens = (int32_t)total;
  const int Hq = desc->num_q_heads, Hkv = desc->num_kv_heads;
  const int G = Hq / Hkv;
  p->group = G;
  // Heads packed per prefill tile: the largest power of two dividing G (it
  // divides the kPrefillRows rows); the tile then holds kPrefillRows/GP queries.
  int GP = 1;
  while (GP < cpa::kPrefillRows && G % (GP * 2) == 0) GP *= 2;
  const int QT = cpa::kPrefillRows / GP;
  const bool decode_kernel = cpa::decode_group_supported(G);
  p->decode_group = decode_kernel ? G : 0;

  std::vector<Tile> tiles;
  std::vector<int32_t> decode_seqs;
  int32_t tok = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t ql = query_lens[s], n = seq_lens[s], hist = n - ql;
    p->visible_pairs += (int64_t)Hq * ((int64_t)ql * hist + (int64_t)ql * (ql + 1) / 2);
    if (ql == 1 && decode_kernel) {
      decode_seqs.push_back(s);
    } else if (ql > 0) {
      for (int g = 0; g < Hkv; ++g)
        for (int hs = 0; hs < G / GP; ++hs)
          for (int q0 = 0; q0 < ql; q0 += QT) {
            const int nq = std::min(QT, ql - q0);
            tiles.push_back(Tile{s, g, g * G + hs * GP, GP, tok + q0, q0, nq, hist, hist + q0 + nq});
          }
    }
    tok += ql;
  }

  // Split long prefill key ranges when the tiles alone cannot give every
  // compute unit one work item (one 8-wave item fills a CU); the piece size
  // is the smallest that keeps all items in a single round. All items then
  // run at once, so the launch lasts about as long as its longest item: the
  // split is kept only if it shortens that item by more tiles than the
  // combine launch costs. Items are also split so none touches more than
  // kPrefillPageCap block-table entries.
  const int cus = opt.num_cus > 0 ? opt.num_cus : cpa::kDefaultCus;
  const int target = opt.target_items > 0 ? opt.target_items : cus;
  const int64_t page_cap_keys =
      ((int64_t)(cpa::kPrefillPageCap - 1) * desc->page_size) / cpa::kSplitAlign * cpa::kSplitAlign;
  int64_t chunk_keys = page_cap_keys;
  if (opt.prefill_split == 0 && (int64_t)tiles.size() < target && !tiles.empty()) {
    int64_t total_keys = 0, longest = 0;
    int max_rows = 0;
    for (const Tile& t : tiles) {
      total_keys += t.kv_len;
      longest = std::max<int64_t>(longest, t.kv_len);
      max_rows = std::max(max_rows, t.nq * t.nheads);
    }
    int64_t c = (int64_t)cpa::round_up((size_t)((total_keys + target - 1) / target),
                                       cpa::kSplitAlign);
    c = std::max<int64_t>(c, std::max(opt.min_split_keys, cpa::kSplitAlign));
    auto count = [&](int64_t ck) {
      int64_t items = 0;
      for (const Tile& t : tiles) items += (t.kv_len + ck - 1) / ck;
      return items;
    };
    while (count(c) > target) c += cpa::kSplitAlign;
    const int64_t tiles_unsplit = (longest + cpa::kSplitAlign - 1) / cpa::kSplitAlign;
    const int64_t combine_tiles = (desc->head_dim == 64 && max_rows <= cpa::kSmallItemRows)
                                      ? 2 * cpa::kCombineTiles
                                      : cpa::kCombineTiles;
    if (opt.min_split_keys > 0 || tiles_unsplit - c / cpa::kSplitAlign > combine_tiles)
      chunk_keys = std::min(chunk_keys, c);
  }
  bool fits = true;
  for (const Tile& t : tiles) {
    int64_t nsplit = (t.kv_len + chunk_keys - 1) / chunk_keys;
    if (opt.prefill_split > 0) nsplit = std::max<int64_t>(nsplit, opt.prefill_split);
    fits = fits && add_split(p, p->prefill, t, nsplit, cpa::kSplitAlign);
  }

  int dsk = opt.decode_split_keys;
  if (dsk <= 0) {
    for (int cand : cpa::kDecodeSplitChoices) {
      dsk = cand;
      int64_t items = 0;
      for (int32_t s : decode_seqs) items += ((int64_t)seq_lens[s] + cand - 1) / cand * Hkv;
      if (items >= (int64_t)cpa::kDecodeItemsPerCu * cus) break;
    }
  }
  std::vector<int32_t> qsl((size_t)num_seqs + 1, 0);
  for (int32_t s = 0; s < num_seqs; ++s) qsl[s + 1] = qsl[s] + query_lens[s];
  for (int32_t s : decode_seqs) {
    const int32_t t0 = qsl[s];
    const int32_t n = seq_lens[s];
    for (int g = 0; g < Hkv; ++g) {
      Tile t{s, g, g * G, G, t0, 0, 1, n - 1, n};
      fits = fits && add_split(p, p->decode, t, ((int64_t)n + dsk - 1) / dsk, 1);
    }
  }
  if (!fits) {
    delete p;
    return cpa::fail(CPA_ERR_UNSUPPORTED,
                     "plan too large: more than " + std::to_string(kMaxPlanItems) +
                         " work items or 2^31 partial rows (raise decode_split_keys or lower "
                         "prefill_split)");
  }
  order_for_xcds(p->prefill, cpa::kNumXcds);
  order_for_xcds(p->decode, cpa::kNumXcds);
  for (const cpa::WorkItem& w : p->prefill)
    p->prefill_max_rows = std::max(p->prefill_max_rows, w.nq * w.nheads);

  // Workspace: [zeros][prefill items][decode items][combine items][partial O][partial m,l]
  size_t off = cpa::kZeroBytes;
  p->off_prefill = off;
  off = cpa::round_up(off + p->prefill.size() * sizeof(cpa::WorkItem), cpa::kAlign);
  p->off_decode = off;
  off = cpa::round_up(off + p->decode.size() * sizeof(cpa::WorkItem), cpa::kAlign);
  p->off_combine = off;
  off = cpa::round_up(off + p->combine.size() * sizeof(cpa::CombineItem), cpa::kAlign);
  p->off_part_o = off;
  // Split partials O/l are kept in the output's precision: bf16 partials
  // halve the bytes the split items write and the combine reads, which
  // shortens every split call measurably (fp32 partials of bf16 outputs
  // cost 8-12 us per Llama-3-8B chunk at H = 4096..12288).
  p->part_bf16 = desc->out_dtype == CPA_DTYPE_BF16;
  const size_t part_elem = p->part_bf16 ? sizeof(uint16_t) : sizeof(float);
  off = cpa::round_up(off + (size_t)p->part_rows * desc->head_dim * part_elem, cpa::kAlign);
  p->off_part_ml = off;
  off = cpa::round_up(off + (size_t)p->part_rows * 2 * sizeof(float), cpa::kAlign);
  p->ws_bytes = std::max(off, cpa::kAlign);

  p->image.assign(p->off_part_o, 0);
  if (!p->prefill.empty())
    std::memcpy(p->image.data() + p->off_prefill, p->prefill.data(),
                p->prefill.size() * sizeof(cpa::WorkItem));
  if (!p->decode.empty())
    std::memcpy(p->image.data() + p->off_decode, p->decode.data(),
                p->decode.size() * sizeof(cpa::WorkItem));
  if (!p->combine.empty())
    std::memcpy(p->image.data() + p->off_combine, p->combine.data(),
                p->combine.size() * sizeof(cpa::CombineItem));
  {
    std::lock_guard<std::mutex> lk(cpa::g_ws_mu);
    p->id = cpa::g_next_plan_id++;
  }
  *out_plan = p;
  *workspace_bytes = p->ws_bytes;
  return cpa::ok();
}

cpa_status cpa_plan_destroy(cpa_plan plan) {
  if (!plan) return cpa::ok();
  {
    std::lock_guard<std::mutex> lk(cpa::g_ws_mu);
    for (auto it = cpa::g_ws_owner.begin(); it != cpa::g_ws_owner.end();) {
      if (it->second == plan->id)
        it = cpa::g_ws_owner.erase(it);
      else
        ++it;
    }
  }
  delete plan;
  return cpa::ok();
}

cpa_status cpa_plan_get_info(cpa_plan plan, cpa_plan_info* info) {
  if (!plan || !info) return cpa::fail(CPA_ERR_INVALID_ARG, "plan_get_info: NULL pointer");
  info->num_seqs = plan->num_seqs;
  info->num_tokens = plan->num_tokens;
  info->num_prefill_items = (int32_t)plan->prefill.size();
  info->num_decode_items = (int32_t)plan->decode.size();
  info->num_combine_items = (int32_t)plan->combine.size();
  info->num_partial_rows = plan->part_rows;
  info->visible_pairs = plan->visible_pairs;
  info->workspace_bytes = plan->ws_bytes;
  return cpa::ok();
}

cpa_status cpa_plan_upload(cpa_plan plan, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!plan || !workspace) return cpa::fail(CPA_ERR_INVALID_ARG, "plan_upload: NULL pointer");
  if (workspace_bytes < plan->ws_bytes)
    return cpa::fail(CPA_ERR_WORKSPACE, "plan_upload: workspace has " +
                                            std::to_string(workspace_bytes) + " bytes, plan needs " +
                                            std::to_string(plan->ws_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % cpa::kAlign != 0)
    return cpa::fail(CPA_ERR_INVALID_ARG, "plan_upload: workspace must be 256-byte aligned");
  if (!plan->image.empty()) {
    const hipError_t e = hipMemcpyAsync(workspace, plan->image.data(), plan->image.size(),
                                        hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return cpa::hip_fail(e, "plan_upload copy");
  }
  std::lock_guard<std::mutex> lk(cpa::g_ws_mu);
  cpa::g_ws_owner[workspace] = plan->id;
  return cpa::ok();
}

cpa_status cpa_attention(cpa_plan plan, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return attention_impl(plan, q, k_cache, v_cache, block_table, out, workspace, workspace_bytes,
                        stream, nullptr);
}

cpa_status cpa_kv_write_attention(cpa_plan plan, const void* q, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping, void* k_cache,
                                  void* v_cache, const int32_t* block_table, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const NewRows nr{k_new, v_new, slot_mapping, k_cache, v_cache};
  return attention_impl(plan, q, k_cache, v_cache, block_table, out, workspace, workspace_bytes,
                        stream, &nr);
}

cpa_status cpa_validate_metadata(const cpa_layer_desc* desc, const int32_t* slot_mapping,
                                 int32_t num_tokens, const int32_t* block_table,
                                 const int32_t* query_lens, const int32_t* seq_lens,
                                 int32_t num_seqs) {
  cpa_status st = cpa::check_desc(desc);
  if (st != CPA_OK) return st;
  const int64_t slots = (int64_t)desc->num_blocks * desc->page_size;
  if (slot_mapping) {
    if (num_tokens < 0) return cpa::fail(CPA_ERR_INVALID_ARG, "num_tokens < 0");
    std::vector<uint8_t> seen((size_t)slots, 0);
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int32_t sl = slot_mapping[t];
      if (sl < 0) continue;
      if (sl >= slots)
        return cpa::fail(CPA_ERR_INVALID_ARG, "slot_mapping[" + std::to_string(t) + "] = " +
                                                  std::to_string(sl) + " is outside the cache");
      if (seen[(size_t)sl]++)
        return cpa::fail(CPA_ERR_INVALID_ARG,
                         "slot_mapping[" + std::to_string(t) + "] repeats slot " + std::to_string(sl));
    }
  }
  if (query_lens && seq_lens) {
    int64_t total = 0;
    st = cpa::check_lens(desc, query_lens, seq_lens, num_seqs, &total);
    if (st != CPA_OK) return st;
    if (slot_mapping && total != num_tokens)
      return cpa::fail(CPA_ERR_INVALID_ARG, "sum(query_lens) != num_tokens");
    if (block_table) {
      for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t pages = ((int64_t)seq_lens[s] + desc->page_size - 1) / desc->page_size;
        for (int64_t j = 0; j < pages; ++j) {
          const int32_t pg = block_table[(size_t)s * desc->max_blocks_per_seq + j];
          if (pg < 0 || pg >= desc->num_blocks)
            return cpa::fail(CPA_ERR_INVALID_ARG, "block_table[" + std::to_string(s) + "][" +
                                                      std::to_string(j) + "] = " +
                                                      std::to_string(pg) + " is outside the cache");
        }
      }
    }
  }
  return cpa::ok();
}

}  // extern "C"

extern "C" cpa_status cpa_split_point(const int32_t* query_lens, int32_t num_seqs, int32_t mode,
                                      double balance_threshold, int32_t length_threshold,
                                      int32_t* seq_split, int32_t* token_split) {
  if (!seq_split || !token_split || num_seqs < 0 || (num_seqs > 0 && !query_lens))
    return cpa::fail(CPA_ERR_INVALID_ARG, "split_point: bad arguments");
  *seq_split = 0;
  *token_split = 0;
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (query_lens[s] < 0) return cpa::fail(CPA_ERR_INVALID_ARG, "split_point: negative query_len");
    total += query_lens[s];
  }
  if (num_seqs < 2) return cpa::ok();  // no split
  if (mode == CPA_SPLIT_SIMPLE) {
    const int32_t k = num_seqs / 2;
    int64_t tsp = 0;
    for (int32_t s = 0; s < k; ++s) tsp += query_lens[s];
    *seq_split = k;
    *token_split = (int32_t)tsp;
    return cpa::ok();
  }
  if (mode != CPA_SPLIT_BALANCED) return cpa::fail(CPA_ERR_INVALID_ARG, "split_point: unknown mode");
  if (!(balance_threshold >= 0.0)) return cpa::fail(CPA_ERR_INVALID_ARG, "split_point: bad threshold");
  const int64_t aim = total / 2;
  int32_t best_k = 0;
  int64_t best_c = 0, cumu = 0;
  for (int32_t k = 1; k < num_seqs; ++k) {
    cumu += query_lens[k - 1];
    const int64_t d = cumu > aim ? cumu - aim : aim - cumu;
    const int64_t db = best_c > aim ? best_c - aim : aim - best_c;
    if (best_k == 0 || d < db) {
      best_k = k;
      best_c = cumu;
    }
  }
  const int64_t n1 = best_c, n2 = total - best_c;
  const int64_t lo = n1 < n2 ? n1 : n2, diff = n1 > n2 ? n1 - n2 : n2 - n1;
  if (lo <= 0) return cpa::ok();
  if ((double)diff / (double)lo > balance_threshold) return cpa::ok();
  if (n1 < length_threshold || n2 < length_threshold) return cpa::ok();
  *seq_split = best_k;
  *token_split = (int32_t)best_c;
  return cpa::ok();
}
