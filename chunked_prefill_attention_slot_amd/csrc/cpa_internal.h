// Internal declarations shared by the host runtime (plan, API) and the
// gfx950 kernels. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace cpa {

// One unit of attention work: query rows [q0, q0+nq) of sequence `seq`
// (flat token tok0 is row q0), query heads [head0, head0+nheads) which all
// read KV head `kvh`, over keys [kv0, kv1). Packed row r of the item is
// query q0 + r / nheads, head head0 + r % nheads. If part >= 0 the item
// writes partials at partial rows part + r instead of the output: O/l
// (0 where l = 0) in the plan's partial precision (AttnArgs::part_bf16),
// and fp32 (max, sum). Read with scalar loads (uniform).
struct WorkItem {
  int32_t seq, kvh, head0, nheads;
  int32_t tok0, q0, nq, hist;
  int32_t kv0, kv1, part, pad;
};
static_assert(sizeof(WorkItem) == 48, "WorkItem layout");

// A tile whose key range was split into nsplit items: partial rows of split
// k are part0 + k*rows + r, r < rows = nq * nheads.
struct CombineItem {
  int32_t tok0, head0, nheads, nq;
  int32_t nsplit, part0, rows, pad;
};
static_assert(sizeof(CombineItem) == 32, "CombineItem layout");

// Everything a kernel needs besides its work list.
struct AttnArgs {
  const uint16_t* q;        // [T, Hq, d] bf16
  const uint16_t* k_cache;  // [NB, Hkv, P, d] bf16
  const uint16_t* v_cache;
  const int32_t* block_table;
  int32_t bt_stride;        // max_blocks_per_seq
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t num_blocks;
  float scale_log2e;        // scale * log2(e): scores go to exp2 directly
  void* out;                // [T, Hq, d] bf16 or fp32
  int32_t out_f32;
  void* part_o;             // [rows, d] split partials O/l: bf16 if part_bf16, else fp32
  int32_t part_bf16;
  float* part_ml;           // [rows, 2] fp32: max (log2 units), sum
  const uint16_t* zeros;    // >= 16 zero bytes: source for keys past a range
  // Fused KV write (prefill kernel only): the step's new K/V rows, their
  // slots and the cache they go to. Keys at positions >= hist of a sequence
  // are then read from k_new / v_new rather than from the cache.
  const uint16_t* k_new;    // [T, Hkv, d] bf16
  const uint16_t* v_new;
  const int32_t* slot_mapping;  // [T]
  uint16_t* k_cache_w;      // the same buffers as k_cache / v_cache
  uint16_t* v_cache_w;
  int32_t num_new_tokens;
};

// Prefill work items: 8 waves of 32 packed rows (query x head) each.
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = 32 * kPrefillWaves;
// Block-table entries one prefill item may touch (staged in LDS).
constexpr int kPrefillPageCap = 2048;
// Key ranges of split items start on multiples of this.
constexpr int kSplitAlign = 64;
// Bytes of zeros at the start of the workspace.
constexpr int kZeroBytes = 256;

// Cache rows one fused prefill thread writes at most (K and V).
constexpr int kFusedWritesPerThread = 4;

// fused: also write the step's new K/V rows into the cache (the AttnArgs
// k_new .. num_new_tokens fields), reading new keys from k_new / v_new.
// max_rows: the largest nq * nheads over the items (small items let waves
// without rows skip their work).
hipError_t launch_prefill(const WorkItem* items, int num_items,
                          const AttnArgs& a, int head_dim, bool fused,
                          int max_rows, hipStream_t stream);
hipError_t launch_decode(const WorkItem* items, int num_items,
                         const AttnArgs& a, int head_dim, int group,
                         hipStream_t stream);
// max_rows / max_splits: the largest rows and nsplit over the items; up to
// 8 splits one thread folds a row's splits, beyond that 2-8 threads share them.
hipError_t launch_combine(const CombineItem* items, int num_items,
                          int max_rows, int max_splits, const AttnArgs& a,
                          int head_dim, hipStream_t stream);
hipError_t launch_kv_write(const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           uint16_t* k_cache, uint16_t* v_cache,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_log2, int32_t num_blocks,
                           hipStream_t stream);

// Decode kernel handles these GQA group sizes; others go to the prefill
// kernel.
inline bool decode_group_supported(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8;
}

}  // namespace cpa
