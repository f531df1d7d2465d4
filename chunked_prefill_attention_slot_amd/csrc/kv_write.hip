// KV write: scatter a chunk's new K/V rows into the paged cache through
// slot_mapping (Ascend dual-stream article, section 3.1: slot_mapping maps
// each token of the flat axis to its cache slot; vLLM chunked-prefill
// article, section 3.1: every chunk caches its KV).
//
// HBM-bound byte copy. One thread moves one 16-byte chunk of K and the
// same chunk of V; consecutive threads take consecutive chunks of a token's
// [Hkv, d] row, so both the reads and the writes are contiguous runs of
// d*2 bytes (one head's row in one page slot).
#include "cpa_internal.h"

namespace cpa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_write_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    int32_t num_kv_heads, int32_t chunks_per_row, int32_t page_log2,
    int64_t num_slots) {
  const int64_t per_token = (int64_t)num_kv_heads * chunks_per_row;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_token * num_tokens) return;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;            // h * chunks + c
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;          // padding / outside cache
  const int64_t page = slot >> page_log2;
  const int64_t off = slot & ((1 << page_log2) - 1);
  const int64_t h = rem / chunks_per_row;
  const int64_t c = rem - h * chunks_per_row;
  const int64_t dst =
      (((page * num_kv_heads + h) << page_log2) + off) * chunks_per_row + c;
  const u32x4 kv = __builtin_nontemporal_load(&k_new[idx]);
  const u32x4 vv = __builtin_nontemporal_load(&v_new[idx]);
  __builtin_nontemporal_store(kv, &k_cache[dst]);
  __builtin_nontemporal_store(vv, &v_cache[dst]);
}

}  // namespace

hipError_t launch_kv_write(const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           uint16_t* k_cache, uint16_t* v_cache,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_log2, int32_t num_blocks,
                           hipStream_t stream) {
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int64_t num_slots = (int64_t)num_blocks << page_log2;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     stream, reinterpret_cast<const u32x4*>(k_new),
                     reinterpret_cast<const u32x4*>(v_new), slot_mapping,
                     num_tokens, reinterpret_cast<u32x4*>(k_cache),
                     reinterpret_cast<u32x4*>(v_cache), num_kv_heads, chunks,
                     page_log2, num_slots);
  return hipGetLastError();
}

}  // namespace cpa
