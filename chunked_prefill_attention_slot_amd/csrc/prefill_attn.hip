// Chunked-prefill attention on bf16 MFMA (gfx950).
//
// What it computes: the vLLM "Chunked-Prefills" article, section 3.2.1 --
// a chunk's queries attend over the cached keys/values concatenated with
// the chunk's own (in the paged cache, or read from the step's new rows in
// the fused mode below), scores scaled and
// softmaxed over keys, then a weighted sum of values -- with the causal
// mask offset by the prefix length H (query row i sits at absolute position
// H+i and sees keys 0..H+i), and the paged-cache metadata of the Ascend
// dual-stream article, section 3.1 (block_table, seq_lens, query_lens).
//
// Work item = 256 packed rows (queries x heads of one GQA group that share
// a KV head) over one key range; eight waves, two per SIMD, so one wave's
// softmax runs on the vector ALU while the other's products run on the
// matrix core. Wave w owns packed rows 32w..32w+31. Per 64-key tile:
//   * K and V rows ([key][d], as in the cache pages) are copied straight
//     from HBM into LDS with global_load_lds_dwordx4 (no register staging),
//     gathered through the block-table entries the item touches (staged in
//     LDS once), over four buffers: tile t+2 is in flight while t is used;
//     16-byte chunks are XOR-swizzled per row to keep the reads below free
//     of bank conflicts;
//   * S^T = K.Q^T on v_mfma_f32_32x32x16_bf16 (K is the A operand from LDS,
//     the wave's Q fragment the B operand kept in registers): each lane then
//     holds the scores of ONE query for 16 keys of every 32-key block, so
//     the row max needs one permlane32 swap, and the bf16 weights already
//     sit in the B-operand layout of the second product;
//   * the causal mask is applied only on tiles that cross the diagonal or
//     the end of the key range (select -inf);
//   * online softmax in fp32 with exp2 against a per-row reference
//     (scale*log2(e) folded into Q): the reference is 0 unless the row's
//     scores leave [-64, 64] (then it is subtracted on the vector ALU), set
//     at the row's first visible key and moved only when a tile's weights
//     sum past 2^64, so a common tile forms no row max and O is rarely
//     rescaled;
//   * O^T += V^T.P^T on the same MFMA; the V^T operand comes from the [key][d]
//     tile with ds_read_b64_tr_b16, which hands each lane four consecutive
//     keys of one d column.
// Q enters and O leaves through LDS (the free tile buffers), so that the
// HBM accesses move whole rows. In the fused mode (FUSED) the kernel also
// writes the step's new K/V rows into the cache and reads every key at a
// position >= H from those rows instead, so no read depends on a write in
// the same launch.
// The rows of K fed to the first product are the tile's keys with bits 2
// and 3 of the index swapped; that makes each lane's eight accumulators of
// one 16-key half-block eight consecutive keys, the order the transposed V
// reads deliver. A contraction does not depend on the order of its terms.
#include <math.h>

#include <type_traits>

#include "cpa_internal.h"

namespace cpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte chunk swizzle of staged Q row r. The eight lanes of one
// ds_read_b128 phase read rows 0..7 at the same logical chunk; these land on
// distinct bank groups (rows of d = 64 are half a bank cycle long).
template <int CPR>
__device__ __forceinline__ int q_swz(int r) {
  if constexpr (CPR == 16) return r & 7;
  return (r >> 1) & 3;
}

template <int D>
struct Cfg {
  static constexpr int NW = kPrefillWaves;
  static constexpr int BN = 64;                // keys per tile
  static constexpr int ROWB = D * 2;           // bytes per key row
  static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;       // bytes of one K (or V) tile
  static constexpr int RPI = 1024 / ROWB;      // rows per wave DMA instruction
  static constexpr int IPW = TILE / 1024 / NW; // DMA instructions per wave per matrix
  static constexpr int NKB = BN / 32;          // 32-key MFMA blocks per tile
  static_assert(NKB == 2, "the row max tree assumes two 32-key blocks");
  static constexpr int NKS = D / 16;           // 16-wide d steps of K.Q^T
  static constexpr int NDB = D / 32;           // 32-row d blocks of V^T.P^T
  static constexpr int NBUF = 4;               // LDS tile buffers
  static constexpr int V_REGION = NBUF * TILE; // V tiles follow the K tiles
  static_assert(IPW >= 1, "tile too small for the wave count");
};

template <int N>
using ic = std::integral_constant<int, N>;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One 16-byte global -> LDS copy per lane: lane i's bytes land at LDS
// address lds + 16*i. Issued through inline assembly so that the compiler
// does not order every later LDS read behind it (it cannot tell the two
// tile buffers apart); completion is awaited explicitly with vmcnt before
// the barrier that publishes a tile.
// m0 (which holds the LDS address) is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// The same copy with a uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (no per-lane address arithmetic).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// 16-byte chunk swizzle of K row r. The eight lanes of one ds_read_b128
// phase read rows {0,1,2,3,8,9,10,11} (+4, +16, +32k) at the same logical
// chunk; these land on distinct bank groups.
template <int CPR>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (CPR == 16) return (r & 3) | ((r >> 1) & 4) | ((r & 4) << 1);
  return (r & 3) | ((r >> 1) & 4);
}
// 16-byte chunk swizzle of V row r. A transposed read by 16 lanes touches
// four consecutive rows at two neighbouring chunks, 32 lanes the same rows
// at four chunks; XOR with 0, 6, 10, 12 (d = 128) spreads either set over
// distinct bank groups (XOR with 0, 2, 4, 6 for the 8-chunk rows of d = 64).
template <int CPR>
__device__ __forceinline__ int v_swz(int r) {
  if constexpr (CPR == 16) return (0xCA60u >> (4 * (r & 3))) & 15;
  return (r & 3) << 1;
}

template <int D, bool FUSED, bool SKIP>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kernel(
    const WorkItem* __restrict__ items, AttnArgs a) {
  using C = Cfg<D>;
  constexpr int NW = C::NW, BN = C::BN, ROWB = C::ROWB, CPR = C::CPR, TILE = C::TILE,
                RPI = C::RPI, IPW = C::IPW, NKB = C::NKB, NKS = C::NKS, NDB = C::NDB,
                V_REGION = C::V_REGION;
  // [K tile 0..2][V tile 0..2]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::NBUF * TILE];
  __shared__ int32_t s_pages[kPrefillPageCap];

  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const float sl2e = a.scale_log2e;

  // This lane's query column: packed row r, of query qi.
  const int r = 32 * w + n;
  const int qi = r / it.nheads;
  const bool row_ok = qi < it.nq;
  // SKIP: a wave whose 32 packed rows all lie past the item's rows (a chunk
  // shorter than the item, a decode row of a 16-head group) keeps only its
  // share of the tile copies, the waits and the barriers, and leaves its
  // SIMD to the partner wave. At d = 128 the test held across the loop
  // costs scalar-register spills (16 -> 23) and slows full items, so the
  // d = 128 kernel takes it in a separate instance, launched only when no
  // item has more than 128 rows.
  const bool busy = !SKIP || 32 * w < it.nq * it.nheads;
  const int qpos = it.hist + it.q0 + qi;

  // Q is copied into LDS first (buffers 2 and 3, which the first tile
  // copies leave free), whole rows per DMA instruction: a direct load in
  // the fragment layout would send each load instruction to 32 rows.
  const uint32_t smem_lds =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int q_region = (w < NW / 2 ? 2 * TILE : V_REGION + 2 * TILE) + (w % (NW / 2)) * 32 * ROWB;
  static_assert((NW / 2) * 32 * ROWB <= 2 * TILE, "Q staging exceeds two tile buffers");
  {
    const int lrow = lane / CPR, lpc = lane % CPR;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int R = k * RPI + lrow;  // row of the wave
      const int rq = 32 * w + R;
      const int q = rq / it.nheads, h = rq - q * it.nheads;
      const uint16_t* src = a.zeros;
      if (q < it.nq)
        src = a.q + ((size_t)(it.tok0 + q) * a.num_q_heads + it.head0 + h) * D +
              (lpc ^ q_swz<CPR>(R)) * 8;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(smem_lds + q_region + k * 1024));
    }
  }
  bf16x8 qf[NKS];
  // Fused KV write: this workgroup's share of the step's new rows (16-byte
  // chunks idx = (blockIdx + k*gridDim)*threads + tid, below 2^31: the host
  // fuses only then), loaded now and stored once the prologue's loads have
  // landed. Nothing in this launch reads them from the cache: keys at
  // positions >= hist come from k_new and v_new.
  constexpr int KVW = FUSED ? kFusedWritesPerThread : 0;
  u32x4 kw_k[KVW > 0 ? KVW : 1], kw_v[KVW > 0 ? KVW : 1];
  int32_t kw_slot[KVW > 0 ? KVW : 1];
  constexpr int CPT = D / 8;  // 16-byte chunks per head row
  const int64_t kw_per_tok = (int64_t)a.num_kv_heads * CPT;
  const int64_t kw_total = kw_per_tok * a.num_new_tokens;
  if constexpr (FUSED) {
#pragma unroll
    for (int k = 0; k < KVW; ++k) {
      const uint32_t idx = (blockIdx.x + k * gridDim.x) * (64 * NW) + tid;
      kw_slot[k] = -1;
      if (idx < (uint32_t)kw_total) {
        kw_slot[k] = a.slot_mapping[idx / (uint32_t)kw_per_tok];
        kw_k[k] = reinterpret_cast<const u32x4*>(a.k_new)[idx];
        kw_v[k] = reinterpret_cast<const u32x4*>(a.v_new)[idx];
      }
    }
  }
  // Stage the block-table entries of this item's key range (the loads
  // overlap the Q copy).
  const int j_end = min(it.kv1, it.hist + it.q0 + it.nq);
  const int plog = a.page_log2, pmask = (1 << plog) - 1;
  const int page0 = it.kv0 >> plog;
  if (it.kv0 < j_end) {
    const int npages = ((j_end - 1) >> plog) - page0 + 1;
    const int32_t* bt = a.block_table + (size_t)it.seq * a.bt_stride + page0;
    for (int i = tid; i < npages; i += 64 * NW) {
      const int32_t pg = bt[i];
      s_pages[i] = ((unsigned)pg < (unsigned)a.num_blocks) ? pg : -1;
    }
  }
  // Q fragment: B operand of K.Q^T, lane holds d = 16ks + 8hh .. +7 of row
  // n, multiplied by scale*log2(e) and rounded to bf16, so the products are
  // scores in log2 units (the rounding perturbs a score by far less than
  // the bf16 rounding of the weights that follows). The wave reads only the
  // rows it copied.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (FUSED) {
    const int64_t num_slots = (int64_t)a.num_blocks << a.page_log2;
#pragma unroll
    for (int k = 0; k < KVW; ++k) {
      const uint32_t idx = (blockIdx.x + k * gridDim.x) * (64 * NW) + tid;
      const int32_t slot = kw_slot[k];
      if (idx < (uint32_t)kw_total && slot >= 0 && slot < num_slots) {
        const uint32_t rem = idx % (uint32_t)kw_per_tok;  // h * CPT + c
        const uint32_t h = rem / CPT, c = rem % CPT;
        const int64_t page = slot >> a.page_log2, off = slot & ((1 << a.page_log2) - 1);
        const int64_t dst = (((page * a.num_kv_heads + h) << a.page_log2) + off) * CPT + c;
        __builtin_nontemporal_store(kw_k[k], reinterpret_cast<u32x4*>(a.k_cache_w) + dst);
        __builtin_nontemporal_store(kw_v[k], reinterpret_cast<u32x4*>(a.v_cache_w) + dst);
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u32x4 qv = *reinterpret_cast<const u32x4*>(
        smem + q_region + n * ROWB + (((2 * ks + hh) ^ q_swz<CPR>(n)) << 4));
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = pack_bf16x2(__uint_as_float(qv[j] << 16) * sl2e,
                         __uint_as_float(qv[j] & 0xFFFF0000u) * sl2e);
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  __syncthreads();

  // DMA of one tile: wave w issues instructions w*IPW + u of each matrix;
  // lane -> (row, physical chunk); keys past j_end read a zero block. The
  // IPW*RPI rows of one wave lie in one page (pages hold >= 16 keys), so the
  // page number is one uniform value per wave, looked up ahead of the copy.
  static_assert(IPW * RPI <= 16, "a wave's rows must fit the smallest page");
  const int lrow = lane / CPR, lpc = lane % CPR;
  // Block-table entry of this wave's rows of the tile at key j0, read from
  // the staged copy; -1 past the key range. page_of makes it uniform. In the
  // tile loop the entry is read one copy ahead, so the read's latency (it
  // queues behind the other waves' operand reads) is not waited for.
  auto page_raw = [&](int j0) __attribute__((always_inline)) -> int {
    const int key_w = j0 + w * IPW * RPI;
    return (key_w < j_end) ? s_pages[(key_w >> plog) - page0] : -1;
  };
  auto page_of = [&](int j0) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(page_raw(j0));
  };
  // Byte offsets of this lane's 16 bytes from the wave's first row (row
  // u*RPI + lrow of the wave's IPW*RPI, chunk swizzled to where it lands).
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int row = (w * IPW + u) * RPI + lrow;  // tile row (same low bits)
    koff[u] = (uint32_t)(((u * RPI + lrow) * D + (lpc ^ k_swz<CPR>(row)) * 8) * 2);
    voff[u] = (uint32_t)(((u * RPI + lrow) * D + (lpc ^ v_swz<CPR>(row)) * 8) * 2);
  }
  // Extra per-lane byte offset of a new-key row in k_new / v_new, whose rows
  // are Hkv*d elements apart instead of d.
  const uint32_t new_xoff = FUSED ? (uint32_t)(lrow * (a.num_kv_heads - 1) * D * 2) : 0u;
  // PARTS selects the matrices copied: 1 = K, 2 = V, 3 = both.
  auto issue = [&](int j0, int pg, int buf, auto parts) __attribute__((always_inline)) {
    constexpr int PARTS = decltype(parts)::value;
    const uint32_t kbuf = smem_lds + buf * TILE;
    const uint32_t vbuf = smem_lds + V_REGION + buf * TILE;
    const int key_w = j0 + w * IPW * RPI;
    // Rows read from the cache end at j_end, or (fused) at the first new key.
    const int lim_c = FUSED ? min(j_end, it.hist) : j_end;
    if (pg >= 0 && key_w + IPW * RPI <= lim_c) {
      // All rows of this wave are in range: uniform page base in SGPRs.
      const size_t e0 = ((((size_t)pg * a.num_kv_heads + it.kvh) << plog) + (key_w & pmask)) * D;
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int i = w * IPW + u;
        if constexpr (PARTS & 1) lds_dma16_s(a.k_cache + e0, koff[u], kbuf + i * 1024);
        if constexpr (PARTS & 2) lds_dma16_s(a.v_cache + e0, voff[u], vbuf + i * 1024);
      }
      return;
    }
    if constexpr (FUSED) {
      if (key_w >= it.hist && key_w + IPW * RPI <= j_end) {
        // All rows are this step's new keys: row key of the sequence is
        // token tok0 - q0 + key - hist of k_new, Hkv*d elements apart. The
        // row offsets within one DMA instruction are per lane (koff + the
        // extra stride), those between instructions uniform.
        const size_t e0 =
            ((size_t)(it.tok0 - it.q0 + key_w - it.hist) * a.num_kv_heads + it.kvh) * D;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
          const int i = w * IPW + u;
          const size_t eu = e0 + (size_t)u * RPI * (a.num_kv_heads - 1) * D;
          if constexpr (PARTS & 1) lds_dma16_s(a.k_new + eu, koff[u] + new_xoff, kbuf + i * 1024);
          if constexpr (PARTS & 2) lds_dma16_s(a.v_new + eu, voff[u] + new_xoff, vbuf + i * 1024);
        }
        return;
      }
    }
    // Last tile of the range, a wave straddling the first new key, or an
    // invalid block-table entry: per-lane sources; rows past j_end read a
    // zero block, so masked keys meet finite values.
    const size_t pbase = ((size_t)(pg < 0 ? 0 : pg) * a.num_kv_heads + it.kvh) << plog;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int i = w * IPW + u;
      const int row = i * RPI + lrow;
      const int key = j0 + row;
      const uint16_t* ks = a.zeros;
      const uint16_t* vs = a.zeros;
      if (FUSED && key < j_end && key >= it.hist) {
        const size_t base =
            ((size_t)(it.tok0 - it.q0 + key - it.hist) * a.num_kv_heads + it.kvh) * D;
        ks = a.k_new + base + (lpc ^ k_swz<CPR>(row)) * 8;
        vs = a.v_new + base + (lpc ^ v_swz<CPR>(row)) * 8;
      } else if (key < j_end && pg >= 0) {
        const size_t base = (pbase + (key & pmask)) * D;
        ks = a.k_cache + base + (lpc ^ k_swz<CPR>(row)) * 8;
        vs = a.v_cache + base + (lpc ^ v_swz<CPR>(row)) * 8;
      }
      if constexpr (PARTS & 1) lds_dma16(ks, __builtin_amdgcn_readfirstlane(kbuf + i * 1024));
      if constexpr (PARTS & 2) lds_dma16(vs, __builtin_amdgcn_readfirstlane(vbuf + i * 1024));
    }
  };


  // Per-lane LDS offsets of the operand reads; the tile buffer and the
  // 32-key block add compile-time constants.
  // K: A-operand row n of a 32-key block is key n with bits 2, 3 swapped;
  // accumulator i of lane half hh then holds key 32kb + 16(i>>3) + 8hh + (i&7).
  const int krow = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  int kofs[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kofs[ks] = krow * ROWB + (((2 * ks + hh) ^ k_swz<CPR>(krow)) << 4);
  // V^T by transposed reads: 16-lane group g covers d 16(g&1) .. +15 of each
  // 32-d block and keys 8(g>>1) + 4u + (s>>2) of each 16-key half block;
  // lane s of the group supplies the address of d 4(s&3) .. +3 of its key.
  const int vg = lane >> 4, vl = lane & 15;
  const int vd_off = 16 * (vg & 1) + 4 * (vl & 3);
  const int vkey_off = 8 * (vg >> 1) + (vl >> 2);
  int vofs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    vofs[db] = V_REGION + vkey_off * ROWB +
               (((4 * db + (vd_off >> 3)) ^ v_swz<CPR>(vkey_off)) << 4) + ((vd_off & 7) << 1);
  const auto* smem3 = (const __attribute__((address_space(3))) uint8_t*)smem;

  // Reference of this row in log2 units: the weights are 2^(score - m_ref).
  // It is 0 unless the row's scores leave [-64, 64] (then the weights would
  // leave the range in which their sums are safe), so for common inputs no
  // subtraction is needed at all; unset before the row's first visible key.
  float m_ref = 0.f;
  bool unset = true;
  float l_run = 0.f;         // this lane's part of the row sum
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  f32x16 sc[NKB];     // scores (log2 units) of the newest tile
  bf16x8 pw[2 * NKB]; // its bf16 weights, held for the next X phase

  // Causal mask offset by H, and the end of the key range. Accumulator i
  // of lane half hh holds key j0 + 32kb + 16(i>>3) + 8hh + (i&7).
  auto mask = [&](int j0) __attribute__((always_inline)) {
    if ((j0 + BN - 1 > it.hist + it.q0) || (j0 + BN > it.kv1)) {
      // key = j0 + 8hh + c with c a compile-time constant per accumulator;
      // the key is visible iff c < lim.
      // Bit select against an arithmetic-shift mask rather than a compare
      // per score: 32 compares would each hold a lane mask in scalar
      // registers.
      const int lim1 = min(qpos + 1, it.kv1) - j0 - 8 * hh - 1;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t m = (uint32_t)((lim1 - (32 * kb + 16 * (i >> 3) + (i & 7))) >> 31);
          uint32_t v;
          asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(v) : "v"(m), "v"(0xFF800000u),
              "v"(__float_as_uint(sc[kb][i])));
          sc[kb][i] = __uint_as_float(v);
        }
    }
  };
  // Row max over both lane halves (same query).
  auto row_max = [&]() __attribute__((always_inline)) -> float {
    // Balanced tree: a written chain of maxima stays serial.
    float m8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      m8[j] = fmaxf(fmaxf(sc[0][2 * j], sc[0][2 * j + 1]), fmaxf(sc[1][2 * j], sc[1][2 * j + 1]));
#pragma unroll
    for (int j = 0; j < 4; ++j) m8[j] = fmaxf(m8[j], m8[j + 4]);
    const float mx = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
  };
  // Set the reference at the row's first visible key (0 when the row max
  // mx, relative to the current reference, lies in [-64, 64], else mx), and
  // move it to the row max when a score exceeds it by more than 32 (rare:
  // O and l are rescaled and this tile's scores shifted). sc holds the
  // scores relative to the current reference.
  auto raise_ref = [&](float mx) __attribute__((always_inline)) {
    const bool need = unset ? (mx > -INFINITY) : (mx > 32.f);
    if (__builtin_amdgcn_ballot_w64(need)) {
      float alpha = 1.f, delta = 0.f;
      if (need) {
        const float m_new = (unset && fabsf(mx) <= 64.f) ? m_ref : m_ref + mx;
        alpha = unset ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        delta = m_ref - m_new;
        m_ref = m_new;
        unset = false;
      }
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] += delta;
    }
  };
  // V^T operand of the product for keys 32kb + 16h2 .. +15 and d block db:
  // two transposed reads of four keys each.
  auto v_read = [&](int base) __attribute__((always_inline)) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem3 + base));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem3 + base + 4 * ROWB));
    const u32x4 av = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                      __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    return __builtin_bit_cast(bf16x8, av);
  };

  // bf16 weights 2^(score - m_ref) of the tile in the B-operand layout of the
  // second product (half block 2kb+h2 of lane half hh: eight consecutive
  // keys), and the sum of the fp32 weights before rounding, in four add
  // chains. The sum uses plain fp32 adds: a dot-product instruction (bf16
  // pairs dotted with ones) does not issue beside the other wave's matrix
  // products and serialised the two wave groups. Summing the unrounded
  // weights is as accurate as summing the rounded ones; constant V then
  // comes back within the bf16 rounding of the weights (relative 2^-8)
  // instead of exactly.
  auto weights = [&](bf16x8 (&pw)[2 * NKB]) __attribute__((always_inline)) -> float {
    float lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x2 pp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(sc[kb][8 * h2 + 2 * j]);
          const float p1 = __builtin_amdgcn_exp2f(sc[kb][8 * h2 + 2 * j + 1]);
          pp[j] = bf16x2{(__bf16)p0, (__bf16)p1};
          lt[j] += p0 + p1;
        }
        const u32x4 w4 = {__builtin_bit_cast(uint32_t, pp[0]), __builtin_bit_cast(uint32_t, pp[1]),
                          __builtin_bit_cast(uint32_t, pp[2]), __builtin_bit_cast(uint32_t, pp[3])};
        pw[2 * kb + h2] = __builtin_bit_cast(bf16x8, w4);
      }
    return (lt[0] + lt[1]) + (lt[2] + lt[3]);
  };

  // X phase: O^T += V^T.P^T for the previous tile (weights pw, V at LDS
  // byte offset vbase) and S^T = K.Q^T for the current tile (K in buffer
  // KB), all on the matrix core. The two score chains and the four O chains
  // are independent, so products issue back to back with the LDS reads
  // running ahead of them. All 16 PV products go first, then the 16 S
  // products: measured ~1.4% faster per step than alternating the two kinds.
  // The first phase of an item has no previous tile (S only) and the last
  // no current tile (PV only).
  auto x_phase = [&](int vbase, auto kbc, auto pvc, auto sc_) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value;
    constexpr bool PV = decltype(pvc)::value, S = decltype(sc_)::value;
    f32x16 acc[NKB];
    if constexpr (S) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) acc[kb] = f32x16{};
    }
#pragma unroll
    for (int i = 0; i < NKB * NKS; ++i) {
      if constexpr (PV) {
        const int hb = i / NDB, db = i % NDB;
        const bf16x8 av = v_read(vofs[db] + vbase + 16 * hb * ROWB);
        oacc[db] = mfma32(av, pw[hb], oacc[db]);
      }
    }
#pragma unroll
    for (int i = 0; i < NKB * NKS; ++i) {
      if constexpr (S) {
        const int kb = i % NKB, ks = i / NKB;
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(smem + (KB * TILE + 32 * kb * ROWB) + kofs[ks]);
        acc[kb] = mfma32(av, qf[ks], acc[kb]);
      }
    }
    if constexpr (S) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[kb] = acc[kb];
    }
    if constexpr (PV && S) {
      __builtin_amdgcn_sched_group_barrier(0x0100, 6, 0);    // DS read
#pragma unroll
      for (int i = 0; i < 2 * NKB * NKS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
        // two transposed V reads per PV product, then one K read per S
        // product, issued ahead of their products
        if (i < NKB * NKS) __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
        else if (i < 2 * NKB * NKS - 4) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
      }
    } else if constexpr (S) {
      __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
      for (int i = 0; i < NKB * NKS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
        if (i + 4 < NKB * NKS) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
      for (int i = 0; i < NKB * NKS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
        if (i + 2 < NKB * NKS) __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
      }
    }
  };

  // Y phase for tile t: mask, then the weights against the current
  // reference. The row max is only formed when a row has no reference yet
  // or when the tile's weights sum past 2^64 (a score more than ~58 above
  // the reference, or NaN from overflow): then the reference moves and the
  // weights are formed again. Otherwise every weight is below 2^64 and its
  // bf16 rounding and fp32 accumulation are as accurate as at any other
  // scale (the two formats share fp32's exponent range), so no max is
  // needed.
  auto y_phase = [&](int t) __attribute__((always_inline)) {
    mask(it.kv0 + t * BN);
    if (__builtin_amdgcn_ballot_w64(m_ref != 0.f)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] -= m_ref;
    }
    float lt = weights(pw);
    if (__builtin_amdgcn_ballot_w64(unset || !(lt <= 0x1p64f))) {
      raise_ref(row_max());
      lt = weights(pw);
    }
    l_run += lt;
  };


  // Two wave groups in ping-pong, half a tile apart. Group 0 (waves
  // 0..NW/2-1) runs X(0) Y(0) X(1) Y(1) ... Y(n-1) X(n), where X(s) is the
  // products PV(s-1) + S(s) and Y(s) the weights of tile s; group 1 runs the
  // same half a tile later. On every SIMD one wave's products thus overlap
  // the other wave's vector work. Tile s lives in LDS buffer s % 4. One
  // barrier per tile, at the start of tile interval s (half steps 2s and
  // 2s+1, in which group 0 runs X(s) Y(s) and group 1 runs Y(s-1) X(s)),
  // after each wave has waited for its copies of tile s: it publishes K(s)
  // for both groups' X(s), and V(s-1) was published one interval earlier.
  // Each wave issues its share of a tile's copy inside a Y phase (group 0
  // copies tile s+2 in Y(s), group 1 copies tile s+2 in Y(s-1)), both in
  // interval s, into the buffer of tile s-2, whose last readers, X(s-2) and
  // X(s-1), finished in earlier intervals. The vector work leaves slack for
  // the copy issue to stall.
  const int grp = w / (NW / 2);
  const int ntiles = (it.kv0 < j_end) ? (j_end - it.kv0 + BN - 1) / BN : 0;
  // Wait until this wave's copy of tile s has landed, leaving the copies of
  // later tiles (at most s+1, or 3 after the prologue) in flight.
  // Every wave has issued its copies of tiles up to s+1 (when they exist)
  // by the time it waits for tile s.
  auto wait_tile = [&](int s) __attribute__((always_inline)) {
    const int ahead = min(ntiles - 1, s + 1) - s;
    if (ahead == 1) {
      if constexpr (IPW == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  if (ntiles > 0) {
    // Tiles 0 and 1 are copied before the loop; the loop copies tile s+2
    // in tile interval s from then on (tile 2 after the X(0) of group 1 and
    // in the Y(0) of group 0).
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (t < ntiles) issue(it.kv0 + t * BN, page_of(it.kv0 + t * BN), t, ic<3>{});
    const int hend = 2 * ntiles;  // the steady half steps are 2 .. hend-1
    // Each group runs its own copy of the loop (same barriers, different
    // phase order), which keeps the register allocation of the two phase
    // sequences apart.
    auto run = [&](auto gc) __attribute__((always_inline)) {
      constexpr int G = decltype(gc)::value;
      // Block-table entry (not yet uniform) for the copy of this wave's next
      // Y phase in the loop: Y(s) copies tile s + 2 + G, the first one tile 3.
      int pg_next = page_raw(it.kv0 + 3 * BN);
      const int pg2 = page_of(it.kv0 + 2 * BN);
      // Half steps 0 and 1: group 0 runs X(0) (scores only) then Y(0);
      // group 1 runs X(0). Both then copy their share of tile 2.
      wait_tile(0);
      __syncthreads();
      if (busy) x_phase(0, ic<0>{}, std::false_type{}, std::true_type{});
      if constexpr (G == 0) {
        if (busy) y_phase(0);
      }
      if (2 < ntiles) issue(it.kv0 + 2 * BN, pg2, 2, ic<3>{});
      // Steady half steps h = 2 .. 2n-1: X(s) with 1 <= s <= n-1, Y(s) with
      // s <= n-1 for either group, buffers known at compile time from h % 8.
      auto half = [&](auto jc, int h) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;  // h % 8
        if constexpr (J % 2 == 0) {
          wait_tile(h >> 1);
          __syncthreads();
        }
        constexpr bool X = ((J - G) & 1) == 0;       // X(s) when h - G is even
        constexpr int SJ = ((J - G + 8) % 8) >> 1;  // s % 4
        const int s = (h - G) >> 1;
        if constexpr (X) {
          if (busy) x_phase(((SJ + 3) % 4) * TILE, ic<SJ>{}, std::true_type{}, std::true_type{});
        } else {
          constexpr int AH = 2 + G;                  // tile copied in this Y phase
          const int tc = s + AH;
          // The copy is issued after the vector work: the issue stalls
          // while the address unit drains the other waves' copies, and the
          // stall then overlaps the wait at the barrier.
          const bool copy = tc < ntiles;
          const int pg = __builtin_amdgcn_readfirstlane(pg_next);
          pg_next = page_raw(it.kv0 + (tc + 1) * BN);
          if (busy) y_phase(s);
          if (copy) issue(it.kv0 + tc * BN, pg, (SJ + AH) % 4, ic<3>{});
        }
      };
      for (int h0 = 2; h0 < hend; h0 += 8) {
        half(ic<2>{}, h0);
        if (h0 + 1 >= hend) break;
        half(ic<3>{}, h0 + 1);
        if (h0 + 2 >= hend) break;
        half(ic<4>{}, h0 + 2);
        if (h0 + 3 >= hend) break;
        half(ic<5>{}, h0 + 3);
        if (h0 + 4 >= hend) break;
        half(ic<6>{}, h0 + 4);
        if (h0 + 5 >= hend) break;
        half(ic<7>{}, h0 + 5);
        if (h0 + 6 >= hend) break;
        half(ic<0>{}, h0 + 6);
        if (h0 + 7 >= hend) break;
        half(ic<1>{}, h0 + 7);
      }
      // Half steps 2n and 2n+1: group 0 runs X(n) (O only, V of tile n-1);
      // group 1 runs Y(n-1) then X(n).
      const int vlast = ((ntiles - 1) & 3) * TILE;
      __syncthreads();
      if constexpr (G == 1) {
        if (busy) y_phase(ntiles - 1);
      }
      if (busy) x_phase(vlast, ic<0>{}, std::true_type{}, std::false_type{});
    };
    if (grp == 0)
      run(ic<0>{});
    else
      run(ic<1>{});
  }

  // Epilogue. Every wave is past its last read of the tile buffers after
  // this barrier; they then stage each wave's O rows, so that the global
  // stores write whole rows (a lane of the accumulator layout holds 4
  // values of one row, and storing from there would send every store
  // instruction to 32 different rows).
  __syncthreads();
  float l_tot;
  {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_tot = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
  }
  // A split item's partial is O/l in the plan's partial precision (a row
  // with no visible key in the range has l = 0 and stores zeros), with fp32
  // (m, l).
  const bool split = it.part >= 0;
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  auto store_rows = [&](auto ec) __attribute__((always_inline)) {
    constexpr int E = decltype(ec)::value;  // bytes per stored element
    constexpr int RB = D * E;               // bytes per row
    constexpr int CH = RB / 16;             // 16-byte chunks per row
    constexpr int RPS = 64 / CH;            // rows per store instruction
    static_assert(NW * 32 * RB <= (int)sizeof(smem), "O staging exceeds the tile buffers");
    uint8_t* region = smem + w * 32 * RB;
    // Lane (n, hh) holds d = 32db + 8g4 + 4hh .. +3 of row n; chunk c of
    // row R sits at chunk c ^ (R mod CH), so neither side conflicts on banks.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int byte = (32 * db + 8 * g4 + 4 * hh) * E;
        uint8_t* dst = region + n * RB + (((byte >> 4) ^ (n & (CH - 1))) << 4) + (byte & 15);
        const float v0 = oacc[db][4 * g4 + 0] * inv, v1 = oacc[db][4 * g4 + 1] * inv;
        const float v2 = oacc[db][4 * g4 + 2] * inv, v3 = oacc[db][4 * g4 + 3] * inv;
        if constexpr (E == 4)
          *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
        else
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
    // The wave reads back only what it wrote; LDS serves one wave's
    // operations in order. The rows go out as streaming stores (nothing in
    // this launch reads them again).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int lr = lane / CH, lc = lane % CH;
#pragma unroll
    for (int k = 0; k < 32 / RPS; ++k) {
      const int R = k * RPS + lr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + R * RB + ((lc ^ (R & (CH - 1))) << 4));
      const int rr = 32 * w + R;  // packed row
      const int q = rr / it.nheads, h = rr - q * it.nheads;
      if (q < it.nq) {
        uint8_t* dst = split
            ? static_cast<uint8_t*>(a.part_o) + ((size_t)it.part + rr) * RB
            : static_cast<uint8_t*>(a.out) +
                  ((size_t)(it.tok0 + q) * a.num_q_heads + it.head0 + h) * RB;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + lc * 16));
      }
    }
  };
  if (split ? !a.part_bf16 : a.out_f32)
    store_rows(ic<4>{});
  else
    store_rows(ic<2>{});
  if (split && hh == 0 && row_ok) {
    float2* ml = reinterpret_cast<float2*>(a.part_ml) + it.part + r;
    *ml = float2{unset ? -INFINITY : m_ref, l_tot};
  }
}

}  // namespace

hipError_t launch_prefill(const WorkItem* items, int num_items, const AttnArgs& a,
                          int head_dim, bool fused, int max_rows, hipStream_t stream) {
  if (num_items == 0) return hipSuccess;
  const dim3 block(64 * kPrefillWaves);
  const dim3 grid(num_items);
  // Items of at most 128 rows leave at least half the waves idle.
  const bool small = max_rows <= kPrefillRows / 2;
  if (head_dim == 128 && fused && small)
    hipLaunchKernelGGL((prefill_kernel<128, true, true>), grid, block, 0, stream, items, a);
  else if (head_dim == 128 && fused)
    hipLaunchKernelGGL((prefill_kernel<128, true, false>), grid, block, 0, stream, items, a);
  else if (head_dim == 128 && small)
    hipLaunchKernelGGL((prefill_kernel<128, false, true>), grid, block, 0, stream, items, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<128, false, false>), grid, block, 0, stream, items, a);
  else if (head_dim == 64 && fused)
    hipLaunchKernelGGL((prefill_kernel<64, true, true>), grid, block, 0, stream, items, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((prefill_kernel<64, false, true>), grid, block, 0, stream, items, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpa
