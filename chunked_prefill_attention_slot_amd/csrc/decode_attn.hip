// Decode rows (query_len = 1) and the split-KV combine.
//
// A decode row is the same attention as a prefill row (vLLM
// "Chunked-Prefills" article, section 3.2.1, one query; Ascend dual-stream
// article, section 3.1: query_len 1, seq_len = prefix + 1), but it reads
// every key and value once for a handful of query heads, so it is bound by
// HBM, not by matrix throughput. This kernel therefore uses plain fp32
// vector arithmetic and spends its effort on the memory stream:
//   * a work item is (sequence, KV head, key range); all G query heads of
//     the GQA group are computed from one read of each K/V row;
//   * d/8 lanes share one key, each loading a 16-byte chunk, so a wave
//     reads whole 256-byte rows (d = 128) out of a page;
//   * each thread keeps U keys' K and V loads in flight before using them;
//   * partial (max, sum, O) of the 16 key slots are merged in registers and
//     LDS; long rows are split over several items and merged by
//     combine_kernel, or combine_wide_kernel past 8 splits (log-sum-exp
//     weights).
#include <math.h>

#include <type_traits>

#include "cpa_internal.h"

namespace cpa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16), left in every lane of
// the group, with DPP moves on the vector ALU: swap neighbours, swap pairs
// (a quad then holds its sum in every lane), mirror each half row (the
// other quad of the eight), mirror the row (the other eight of the 16).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                           decltype(ctrl)::value, 0xF, 0xF, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
  if constexpr (N >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
  return x;
}

// Merge (m2, l2, o2) into (m, l, o); m in log2 units, -inf = empty.
template <int N>
__device__ __forceinline__ void lse_merge(float& m, float& l, float* o, float m2, float l2,
                                          const float* o2) {
  const float mm = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mm);
  const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  m = mm;
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(const WorkItem* __restrict__ items,
                                                     AttnArgs a) {
  constexpr int LPK = D / 8;      // lanes per key
  constexpr int KPW = 64 / LPK;   // keys per wave step
  constexpr int KPB = 4 * KPW;    // keys per block step
  constexpr int U = (G >= 8) ? 4 : (G == 1 ? 16 : 8);  // block steps loaded before use
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ __attribute__((aligned(16))) float s_o[4][G][D];

  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane % LPK, ks = lane / LPK;
  const float sl2e = a.scale_log2e;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const u32x4 q4 = *reinterpret_cast<const u32x4*>(
        a.q + ((size_t)it.tok0 * a.num_q_heads + it.head0 + g) * D + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[g][2 * j] = bf16_lo(q4[j]);
      qv[g][2 * j + 1] = bf16_hi(q4[j]);
    }
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }

  const int32_t* bt = a.block_table + (size_t)it.seq * a.bt_stride;
  const int plog = a.page_log2, pmask = (1 << plog) - 1;
  const size_t head_off = (size_t)it.kvh << plog;

  // Block-table entries of this lane's keys, read one iteration ahead of
  // the K/V loads that use them, so an iteration costs one round trip to
  // memory instead of two.
  auto pages_of = [&](int base, int (&pg)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPB + w * KPW + ks;
      pg[u] = (key < it.kv1) ? bt[key >> plog] : -1;
    }
  };
  int pg_cur[U];
  pages_of(it.kv0, pg_cur);
  for (int base = it.kv0; base < it.kv1; base += U * KPB) {
    u32x4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPB + w * KPW + ks;
      ok[u] = key < it.kv1;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (ok[u]) {
        const int page = pg_cur[u];
        if ((unsigned)page < (unsigned)a.num_blocks) {
          const size_t off =
              (((size_t)page * a.num_kv_heads << plog) + head_off + (key & pmask)) * D + 8 * c;
          kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k_cache + off));
          vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v_cache + off));
        }
      }
      kr[u] = kv;
      vr[u] = vv;
    }
    pages_of(base + U * KPB, pg_cur);

    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kf[2 * j] = bf16_lo(kr[u][j]);
        kf[2 * j + 1] = bf16_hi(kr[u][j]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qv[g][e], kf[e], acc);
        acc = group_sum<LPK>(acc);
        s[u][g] = ok[u] ? acc * sl2e : -INFINITY;
      }
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      const float msc = (mx == -INFINITY) ? 0.f : mx;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - msc);
      float psum = 0.f;
      float p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(s[u][g] - msc);
        psum += p[u];
      }
      l[g] = fmaf(l[g], alpha, psum);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[g][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t wv = vr[u][e >> 1];
          acc = fmaf(p[u], (e & 1) ? bf16_hi(wv) : bf16_lo(wv), acc);
        }
        o[g][e] = acc;
      }
      m[g] = mx;
    }
  }

  // Merge the KPW key slots of the wave (lanes with equal c).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[g][e], off);
      const float m2 = __shfl_xor(m[g], off);
      const float l2 = __shfl_xor(l[g], off);
      lse_merge<8>(m[g], l[g], o[g], m2, l2, o2);
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[w][g][8 * c + e] = o[g][e];
      if (c == 0) {
        s_m[w][g] = m[g];
        s_l[w][g] = l[g];
      }
    }
  }
  __syncthreads();

  // Merge the four waves: thread -> (head g, 4 consecutive d).
  constexpr int D4 = D / 4;
  if (tid < G * D4) {
    const int g = tid / D4, d = 4 * (tid % D4);
    float mm = -INFINITY, ll = 0.f, oo[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float o2[4] = {s_o[ww][g][d], s_o[ww][g][d + 1], s_o[ww][g][d + 2],
                           s_o[ww][g][d + 3]};
      lse_merge<4>(mm, ll, oo, s_m[ww][g], s_l[ww][g], o2);
    }
    if (it.part < 0) {
      const float inv = 1.f / ll;
      const size_t ob = ((size_t)it.tok0 * a.num_q_heads + it.head0 + g) * D + d;
      if (a.out_f32) {
        f32x4 o4 = {oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob) = o4;
      } else {
        u32x2 o2 = {pack_bf16x2(oo[0] * inv, oo[1] * inv), pack_bf16x2(oo[2] * inv, oo[3] * inv)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + ob) = o2;
      }
    } else {
      // Partial of a split key range: O/l in the plan's partial precision.
      const size_t prow = (size_t)it.part + g;
      const float inv = (ll > 0.f) ? 1.f / ll : 0.f;
      if (a.part_bf16) {
        u32x2 o2 = {pack_bf16x2(oo[0] * inv, oo[1] * inv), pack_bf16x2(oo[2] * inv, oo[3] * inv)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.part_o) + prow * D + d) = o2;
      } else {
        f32x4 o4 = {oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.part_o) + prow * D + d) = o4;
      }
      if (d == 0) {
        a.part_ml[prow * 2 + 0] = mm;
        a.part_ml[prow * 2 + 1] = ll;
      }
    }
  }
}

// Log-sum-exp merge of the split partials of one tile. Split k holds
// O_k/l_k (bf16 if PB16, else fp32), max m_k and sum l_k; O = sum_k
// 2^(m_k - m) l_k (O_k/l_k) / sum_k 2^(m_k - m) l_k, m = max_k m_k.
//
// fold_splits adds splits [k0, k1) of tile `it`, for packed row r and the 8
// values from d, to a running (mm, ll, o0, o1): ll = sum 2^(m_k - mm) l_k
// and o the same sum of weighted O_k. B splits are read per batch, every
// load of a batch issued before any is used (indices past k1 - 1 repeat it
// and get weight 0), so a batch costs one round trip to memory; earlier
// batches are rescaled to the running max. A split's (max, sum) pair is one
// 8-byte load, its 8 values one 16-byte load (bf16) or two (fp32).
template <int D, bool PB16, int B>
__device__ __forceinline__ void fold_splits(const CombineItem& it, const AttnArgs& a, int r, int d,
                                            int k0, int k1, float& mm, float& ll, f32x4& o0,
                                            f32x4& o1) {
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  for (int kb = k0; kb < k1; kb += B) {
    float2 mlk[B];
    f32x4 ok0[B], ok1[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int k = min(kb + j, k1 - 1);
      const size_t prow = (size_t)it.part0 + (size_t)k * it.rows + r;
      mlk[j] = ml[prow];
      if constexpr (PB16) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.part_o) +
                                                         prow * D + d);
        ok0[j] = f32x4{bf16_lo(b[0]), bf16_hi(b[0]), bf16_lo(b[1]), bf16_hi(b[1])};
        ok1[j] = f32x4{bf16_lo(b[2]), bf16_hi(b[2]), bf16_lo(b[3]), bf16_hi(b[3])};
      } else {
        const f32x4* po =
            reinterpret_cast<const f32x4*>(static_cast<const float*>(a.part_o) + prow * D + d);
        ok0[j] = po[0];
        ok1[j] = po[1];
      }
    }
    float bm = mm;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (kb + j >= k1) mlk[j].x = -INFINITY;
      bm = fmaxf(bm, mlk[j].x);
    }
    const float a0 = (mm == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mm - bm);
    ll *= a0;
    o0 *= a0;
    o1 *= a0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      // Weight of split k: its sum l_k scaled to the common max; the stored
      // partial is O_k / l_k.
      const float wk =
          (mlk[j].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mlk[j].x - bm) * mlk[j].y;
      ll += wk;
      o0 += wk * ok0[j];
      o1 += wk * ok1[j];
    }
    mm = bm;
  }
}

// O = o / ll into the output row of packed row r (values d .. d+7). F32
// selects the output's precision. Streaming stores: nothing in this launch
// reads the rows again.
template <int D, bool F32>
__device__ __forceinline__ void store_merged(const CombineItem& it, const AttnArgs& a, int r, int d,
                                             float ll, f32x4 o0, f32x4 o1) {
  const float inv = 1.f / ll;
  const int qi = r / it.nheads, hl = r - qi * it.nheads;
  const size_t ob = ((size_t)(it.tok0 + qi) * a.num_q_heads + it.head0 + hl) * D + d;
  if constexpr (F32) {
    f32x4* po = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob);
    __builtin_nontemporal_store(o0 * inv, po);
    __builtin_nontemporal_store(o1 * inv, po + 1);
  } else {
    const u32x4 o = {pack_bf16x2(o0[0] * inv, o0[1] * inv), pack_bf16x2(o0[2] * inv, o0[3] * inv),
                     pack_bf16x2(o1[0] * inv, o1[1] * inv), pack_bf16x2(o1[2] * inv, o1[3] * inv)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + ob));
  }
}

// Tiles with at most B splits (B = 4 or 8): thread -> (packed row r, 8
// consecutive values), all splits in one batch.
template <int D, bool F32, bool PB16, int B>
__global__ __launch_bounds__(256) void combine_kernel(const CombineItem* __restrict__ items,
                                                      AttnArgs a) {
  constexpr int D8 = D / 8;
  const CombineItem it = items[blockIdx.x];
  const int idx = blockIdx.y * 256 + threadIdx.x;
  const int r = idx / D8, d = 8 * (idx % D8);
  if (r >= it.rows) return;
  float mm = -INFINITY, ll = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  fold_splits<D, PB16, B>(it, a, r, d, 0, it.nsplit, mm, ll, o0, o1);
  store_merged<D, F32>(it, a, r, d, ll, o0, o1);
}

// Tiles with more than 8 splits (short chunks over long prefixes, long
// decode rows): S threads share each (packed row, 8 values), each folding
// one contiguous range of the splits, and their (m, l, O) meet in LDS,
// where the first of them merges and stores. S = 2, 4 or 8 for up to 16,
// 32 or more splits, so a group folds one batch of 8 up to 64 splits; one
// thread walking all the splits would pay one memory round trip per batch
// in sequence, and more groups than batches only multiply the blocks.
template <int D, int S>
constexpr int wide_rows_per_block() { return 256 / S / (D / 8); }

template <int D, bool F32, bool PB16, int S>
__global__ __launch_bounds__(256) void combine_wide_kernel(const CombineItem* __restrict__ items,
                                                           AttnArgs a) {
  constexpr int D8 = D / 8, GT = 256 / S, RPB = wide_rows_per_block<D, S>();
  static_assert(GT % D8 == 0 && RPB >= 1, "combine_wide_kernel thread layout");
  __shared__ float s_m[256], s_l[256];
  __shared__ f32x4 s_o0[256], s_o1[256];
  const CombineItem it = items[blockIdx.x];
  const int t = threadIdx.x, g = t / GT, lt = t % GT;
  const int r = blockIdx.y * RPB + lt / D8, d = 8 * (lt % D8);
  const bool valid = r < it.rows;
  const int per = (it.nsplit + S - 1) / S;
  const int k0 = min(g * per, it.nsplit), k1 = min(k0 + per, it.nsplit);
  float mm = -INFINITY, ll = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  if (valid && k0 < k1) fold_splits<D, PB16, 8>(it, a, r, d, k0, k1, mm, ll, o0, o1);
  s_m[t] = mm;
  s_l[t] = ll;
  s_o0[t] = o0;
  s_o1[t] = o1;
  __syncthreads();
  if (g != 0 || !valid) return;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < S; ++j) m = fmaxf(m, s_m[j * GT + lt]);
  float l = 0.f;
  f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const float mj = s_m[j * GT + lt];
    const float wj = (mj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mj - m);
    l += wj * s_l[j * GT + lt];
    p0 += wj * s_o0[j * GT + lt];
    p1 += wj * s_o1[j * GT + lt];
  }
  store_merged<D, F32>(it, a, r, d, l, p0, p1);
}

template <int D>
hipError_t launch_decode_d(const WorkItem* items, int n, const AttnArgs& a, int group,
                           hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), dim3(n), dim3(256), 0, s, items, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), dim3(n), dim3(256), 0, s, items, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4>), dim3(n), dim3(256), 0, s, items, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8>), dim3(n), dim3(256), 0, s, items, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool F32, bool PB16>
hipError_t launch_combine_t(const CombineItem* items, int num_items, int max_rows, int max_splits,
                            const AttnArgs& a, hipStream_t s) {
  auto wide = [&](auto sc) {
    constexpr int S = decltype(sc)::value, RPB = wide_rows_per_block<D, S>();
    const dim3 grid(num_items, (max_rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((combine_wide_kernel<D, F32, PB16, S>), grid, dim3(256), 0, s, items, a);
    return hipGetLastError();
  };
  if (max_splits > 32) return wide(std::integral_constant<int, 8>{});
  if (max_splits > 16) return wide(std::integral_constant<int, 4>{});
  if (max_splits > 8) return wide(std::integral_constant<int, 2>{});
  const int threads = max_rows * (D / 8);
  const dim3 grid(num_items, (threads + 255) / 256);
  if (max_splits <= 4)
    hipLaunchKernelGGL((combine_kernel<D, F32, PB16, 4>), grid, dim3(256), 0, s, items, a);
  else
    hipLaunchKernelGGL((combine_kernel<D, F32, PB16, 8>), grid, dim3(256), 0, s, items, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine_d(const CombineItem* items, int n, int max_rows, int max_splits,
                            const AttnArgs& a, hipStream_t s) {
  if (a.out_f32 && a.part_bf16) return launch_combine_t<D, true, true>(items, n, max_rows, max_splits, a, s);
  if (a.out_f32) return launch_combine_t<D, true, false>(items, n, max_rows, max_splits, a, s);
  if (a.part_bf16) return launch_combine_t<D, false, true>(items, n, max_rows, max_splits, a, s);
  return launch_combine_t<D, false, false>(items, n, max_rows, max_splits, a, s);
}

}  // namespace

hipError_t launch_decode(const WorkItem* items, int num_items, const AttnArgs& a, int head_dim,
                         int group, hipStream_t stream) {
  if (num_items == 0) return hipSuccess;
  if (head_dim == 128) return launch_decode_d<128>(items, num_items, a, group, stream);
  if (head_dim == 64) return launch_decode_d<64>(items, num_items, a, group, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineItem* items, int num_items, int max_rows, int max_splits,
                          const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (num_items == 0) return hipSuccess;
  if (head_dim == 128) return launch_combine_d<128>(items, num_items, max_rows, max_splits, a, stream);
  if (head_dim == 64) return launch_combine_d<64>(items, num_items, max_rows, max_splits, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpa
