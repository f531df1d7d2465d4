// Chunked-prefill attention on bf16 MFMA (gfx950).
//
// What it computes: the vLLM "Chunked-Prefills" article, section 3.2.1 --
// a chunk's queries attend over the cached keys/values concatenated with
// the chunk's own (all already in the paged cache), scores scaled and
// softmaxed over keys, then a weighted sum of values -- with the causal
// mask offset by the prefix length H (query row i sits at absolute position
// H+i and sees keys 0..H+i), and the paged-cache metadata of the Ascend
// dual-stream article, section 3.1 (block_table, seq_lens, query_lens).
//
// Work item = 128 packed rows (queries x heads of one GQA group that share
// a KV head) over one key range. Four waves; wave w owns packed rows
// 32w..32w+31. Per 64-key tile (128 keys when d = 64):
//   * K rows are staged in LDS as [key][d] (16-byte chunks XOR-swizzled),
//     V as [d][key] (8-byte quads XOR-swizzled), both gathered through
//     block_table by all 256 threads with 16-byte loads, prefetched into
//     registers one tile ahead;
//   * S^T = K.Q^T on v_mfma_f32_32x32x16_bf16 (K is the A operand from LDS,
//     the wave's Q fragment the B operand kept in registers), so that each
//     lane ends up holding scores of ONE query for 16 keys per 32-key
//     block: the row max needs one cross-lane swap, and the bf16 P values
//     already sit in the B-operand layout of the next product;
//   * the causal mask is applied only on tiles that cross the diagonal or
//     the end of the key range (select -inf);
//   * online softmax in fp32 with exp2 (scale*log2(e) folded into one FMA);
//   * O^T += V^T.P^T on the same MFMA (V^T from LDS, P^T from registers).
// The order of keys inside a tile is permuted consistently between the K
// rows fed to the first product and the V slots read for the second one;
// a contraction does not depend on the order of its terms.
#include <math.h>

#include "cpa_internal.h"

namespace cpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct Tile {
  static constexpr int CH = D / 8;        // 16-byte chunks per key row
  static constexpr int RPP = 256 / CH;    // key rows per load pass
  static constexpr int BN = 4 * RPP;      // keys per tile (each thread: 4)
  static constexpr int NKB = BN / 32;     // 32-key MFMA blocks per tile
  static constexpr int NKS = D / 16;      // 16-wide d steps of K.Q^T
  static constexpr int NDB = D / 32;      // 32-row d blocks of V^T.P^T
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = D * BN * 2;
  static constexpr int RPP_LOG2 = (RPP == 16) ? 4 : 5;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Swizzle of the 16-byte chunk index of K row r: spreads the 8 rows one
// ds_read_b128 phase touches over distinct bank groups.
template <int RPP_LOG2>
__device__ __forceinline__ int k_swz(int r) {
  return ((r >> RPP_LOG2) & 3) | ((r & 1) << 2);
}
// Swizzle of the 8-byte key-quad index of V^T row d.
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 15; }

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(
    const WorkItem* __restrict__ items, AttnArgs a) {
  using TL = Tile<D>;
  constexpr int CH = TL::CH, RPP = TL::RPP, BN = TL::BN, NKB = TL::NKB,
                NKS = TL::NKS, NDB = TL::NDB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[TL::K_BYTES + TL::V_BYTES];
  uint8_t* const Ks = smem;
  uint8_t* const Vt = smem + TL::K_BYTES;

  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const float sl2e = a.scale_log2e;

  // This lane's query column: packed row r -> (query qi, head hl).
  const int r = 32 * w + n;
  const int qi = r / it.nheads;
  const int hl = r - qi * it.nheads;
  const bool row_ok = qi < it.nq;
  const int qpos = it.hist + it.q0 + qi;

  // Q fragment: B operand of K.Q^T, lane holds d = 16ks + 8hh .. +7.
  bf16x8 qf[NKS];
  {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(
        a.q + ((size_t)(it.tok0 + qi) * a.num_q_heads + it.head0 + hl) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = qrow[2 * ks + hh];
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Loader: thread owns 16-byte chunk lc of key rows lr0 + RPP*p, p < 4.
  const int lc = tid % CH, lr0 = tid / CH;
  const int32_t* bt = a.block_table + (size_t)it.seq * a.bt_stride;
  const int plog = a.page_log2;
  const int pmask = (1 << plog) - 1;
  const int j_end = min(it.kv1, it.hist + it.q0 + it.nq);
  u32x4 kr[4], vr[4];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = j0 + lr0 + RPP * p;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < j_end) {
        const int page = bt[key >> plog];
        if ((unsigned)page < (unsigned)a.num_blocks) {
          const size_t off =
              ((((size_t)page * a.num_kv_heads + it.kvh) << plog) + (key & pmask)) * D +
              (size_t)lc * 8;
          kv = *reinterpret_cast<const u32x4*>(a.k_cache + off);
          vv = *reinterpret_cast<const u32x4*>(a.v_cache + off);
        }
      }
      kr[p] = kv;
      vr[p] = vv;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = lr0 + RPP * p;
      *reinterpret_cast<u32x4*>(Ks + row * (D * 2) +
                                ((lc ^ k_swz<TL::RPP_LOG2>(row)) * 16)) = kr[p];
    }
    // V^T: key lr0 + RPP*p goes to slot 4*lr0 + p of row d.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      const int wd = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (vr[0][wd] >> 16) | (vr[1][wd] & 0xFFFF0000u);
        hi = (vr[2][wd] >> 16) | (vr[3][wd] & 0xFFFF0000u);
      } else {
        lo = (vr[0][wd] & 0xFFFFu) | (vr[1][wd] << 16);
        hi = (vr[2][wd] & 0xFFFFu) | (vr[3][wd] << 16);
      }
      u32x2 q2 = {lo, hi};
      *reinterpret_cast<u32x2*>(Vt + d * (BN * 2) + ((lr0 ^ v_swz(d)) * 8)) = q2;
    }
  };

  float m_run = -INFINITY;  // running max of raw scores of this row
  float l_run = 0.f;        // this lane's part of the running sum
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  // A-operand row of K.Q^T for MFMA row m = n: key 8kb + 4(m>>4) +
  // 2((m>>3)&1) + ((m>>2)&1) + RPP*(m&3). Accumulator i of lane half hh then
  // holds key 8kb + 2(i>>2) + hh + RPP*(i&3).
  const int krow0 = 4 * (n >> 4) + 2 * ((n >> 3) & 1) + ((n >> 2) & 1) + RPP * (n & 3);

  if (it.kv0 < j_end) load_tile(it.kv0);
  for (int j0 = it.kv0; j0 < j_end; j0 += BN) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j0 + BN < j_end) load_tile(j0 + BN);

    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      const int row = krow0 + 8 * kb;
      const uint8_t* kp = Ks + row * (D * 2);
      const int sw = k_swz<TL::RPP_LOG2>(row);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(kp + (((2 * ks + hh) ^ sw) * 16));
        sacc[kb] = mfma32(av, qf[ks], sacc[kb]);
      }
    }

    // Causal mask offset by H, and the end of the key range.
    const bool need_mask = (j0 + BN - 1 > it.hist + it.q0) || (j0 + BN > it.kv1);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 8 * kb + 2 * (i >> 2) + hh + RPP * (i & 3);
          if (!(key <= qpos && key < it.kv1)) sacc[kb][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float msc = (m_new == -INFINITY) ? 0.f : m_new * sl2e;
    const float alpha = __builtin_amdgcn_exp2f(m_run * sl2e - msc);
    m_run = m_new;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sacc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], sl2e, -msc));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // The row sum adds the same bf16-rounded weights the second product
    // multiplies, so every output row is an exact convex combination of V.
    float lsum = 0.f;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 pw;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pw[j] = pack_bf16x2(sacc[kb][8 * h2 + 2 * j], sacc[kb][8 * h2 + 2 * j + 1]);
          lsum += __uint_as_float(pw[j] << 16) + __uint_as_float(pw[j] & 0xFFFF0000u);
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const int b0 = 8 * kb + 4 * h2 + hh;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + n;
          const uint8_t* vp = Vt + d * (BN * 2);
          const int sw = v_swz(d);
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vp + ((b0 ^ sw) * 8));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + (((b0 + 2) ^ sw) * 8));
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = mfma32(__builtin_bit_cast(bf16x8, av), pb, oacc[db]);
        }
      }
    l_run = fmaf(l_run, alpha, lsum);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  if (it.part < 0) {
    const float inv = 1.f / l_tot;
    const size_t ob = ((size_t)(it.tok0 + qi) * a.num_q_heads + it.head0 + hl) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const float v0 = oacc[db][4 * g4 + 0] * inv, v1 = oacc[db][4 * g4 + 1] * inv;
        const float v2 = oacc[db][4 * g4 + 2] * inv, v3 = oacc[db][4 * g4 + 3] * inv;
        if (a.out_f32) {
          f32x4 o4 = {v0, v1, v2, v3};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob + d) = o4;
        } else {
          u32x2 o2 = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + ob + d) = o2;
        }
      }
  } else {
    const size_t prow = (size_t)it.part + r;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        f32x4 o4 = {oacc[db][4 * g4 + 0], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                    oacc[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(a.part_o + prow * D + d) = o4;
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = (m_run == -INFINITY) ? -INFINITY : m_run * sl2e;
      a.part_ml[prow * 2 + 1] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const WorkItem* items, int num_items, const AttnArgs& a,
                          int head_dim, hipStream_t stream) {
  if (num_items == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(num_items), dim3(256), 0, stream, items, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(num_items), dim3(256), 0, stream, items, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpa
