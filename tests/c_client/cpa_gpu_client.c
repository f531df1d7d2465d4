/*
 * A plain C11 client that runs the fused KV write + attention on the GPU
 * through libcpa and the HIP runtime alone (no Python, no torch):
 *
 *   cpa_gpu_client <inputs> <outputs>
 *
 * <inputs>: int32 header {Hq, Hkv, d, P, num_blocks, max_blocks_per_seq,
 * num_seqs, num_tokens}, then query_lens[S], seq_lens[S],
 * block_table[S * max_blocks], slot_mapping[T] (int32), then q[T*Hq*d],
 * k_new[T*Hkv*d], v_new[T*Hkv*d], k_cache[NB*Hkv*P*d], v_cache (bf16 bits).
 * <outputs>: out[T*Hq*d] (bf16 bits), then k_cache and v_cache after the
 * call. Exits non-zero with a message on any error.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "cpa.h"

#define HIP(call)                                                           \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CPA(call)                                                           \
  do {                                                                      \
    if ((call) != CPA_OK) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, cpa_last_error());                 \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int to_device(void** dev, const void* host, size_t bytes) {
  if (hipMalloc(dev, bytes ? bytes : 16) != hipSuccess) return 0;
  return !bytes || hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) == hipSuccess;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <inputs> <outputs>\n", argv[0]);
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  int32_t h[8];
  if (!f || fread(h, sizeof h, 1, f) != 1) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  const int32_t hq = h[0], hkv = h[1], d = h[2], P = h[3], nb = h[4], mb = h[5], S = h[6],
                T = h[7];
  const size_t n_q = (size_t)T * hq * d, n_new = (size_t)T * hkv * d,
               n_cache = (size_t)nb * hkv * P * d;
  int32_t* ql = read_block(f, sizeof(int32_t) * S);
  int32_t* sl = read_block(f, sizeof(int32_t) * S);
  int32_t* bt = read_block(f, sizeof(int32_t) * S * mb);
  int32_t* sm = read_block(f, sizeof(int32_t) * T);
  uint16_t* q = read_block(f, 2 * n_q);
  uint16_t* kn = read_block(f, 2 * n_new);
  uint16_t* vn = read_block(f, 2 * n_new);
  uint16_t* kc = read_block(f, 2 * n_cache);
  uint16_t* vc = read_block(f, 2 * n_cache);
  fclose(f);
  if (!ql || !sl || !bt || !sm || !q || !kn || !vn || !kc || !vc) {
    fprintf(stderr, "short input file\n");
    return 1;
  }

  const cpa_layer_desc desc = {hq, hkv, d, P, nb, mb, (float)(1.0 / sqrt((double)d)), 0};
  cpa_plan plan = NULL;
  size_t ws_bytes = 0;
  CPA(cpa_plan_create(&desc, ql, sl, S, NULL, &plan, &ws_bytes));

  void *d_q, *d_kn, *d_vn, *d_kc, *d_vc, *d_sm, *d_bt, *d_out, *d_ws;
  if (!to_device(&d_q, q, 2 * n_q) || !to_device(&d_kn, kn, 2 * n_new) ||
      !to_device(&d_vn, vn, 2 * n_new) || !to_device(&d_kc, kc, 2 * n_cache) ||
      !to_device(&d_vc, vc, 2 * n_cache) || !to_device(&d_sm, sm, sizeof(int32_t) * T) ||
      !to_device(&d_bt, bt, sizeof(int32_t) * S * mb)) {
    fprintf(stderr, "device copy failed\n");
    return 2;
  }
  HIP(hipMalloc(&d_out, n_q ? 2 * n_q : 16));
  HIP(hipMalloc(&d_ws, ws_bytes));
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  CPA(cpa_plan_upload(plan, d_ws, ws_bytes, stream));
  CPA(cpa_kv_write_attention(plan, d_q, d_kn, d_vn, (const int32_t*)d_sm, d_kc, d_vc,
                             (const int32_t*)d_bt, d_out, d_ws, ws_bytes, stream));
  HIP(hipStreamSynchronize(stream));

  uint16_t* out = malloc(n_q ? 2 * n_q : 16);
  HIP(hipMemcpy(out, d_out, 2 * n_q, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(kc, d_kc, 2 * n_cache, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(vc, d_vc, 2 * n_cache, hipMemcpyDeviceToHost));
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(out, 2, n_q, o) != n_q || fwrite(kc, 2, n_cache, o) != n_cache ||
      fwrite(vc, 2, n_cache, o) != n_cache) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(o);
  CPA(cpa_plan_destroy(plan));
  HIP(hipStreamDestroy(stream));
  void* bufs[] = {d_q, d_kn, d_vn, d_kc, d_vc, d_sm, d_bt, d_out, d_ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP(hipFree(bufs[i]));
  printf("done\n");
  return 0;
}
