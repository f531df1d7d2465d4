// cpa_kv_write_attention_static: the fused KV write + attention call for
// callers that cannot allocate device memory. Its workspace (plan work
// lists, zero bytes, split partials) is a static device array of fixed
// size, one copy per GPU, held until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once
// per device with that device current, and that address is what the
// kernels and the upload copy receive.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "cpa.h"
#include "cpa_host.h"
#include "cpa_internal.h"

namespace cpa {
namespace {

static_assert(CPA_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[CPA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the
// first call on that device).
cpa_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CPA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CPA_ERR_UNSUPPORTED, "static scratch: device index " + std::to_string(dev) +
                                         " out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(CPA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                   hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CPA_OK;
}

}  // namespace
}  // namespace cpa

extern "C" cpa_status cpa_kv_write_attention_static(cpa_plan plan, const void* q,
                                                    const void* k_new, const void* v_new,
                                                    const int32_t* slot_mapping, void* k_cache,
                                                    void* v_cache, const int32_t* block_table,
                                                    void* out, hipStream_t stream) {
  if (!plan) return cpa::fail(CPA_ERR_INVALID_ARG, "kv_write_attention_static: plan is NULL");
  const size_t need = cpa::plan_workspace_bytes(plan);
  if (need > CPA_STATIC_SCRATCH_BYTES)
    return cpa::fail(CPA_ERR_WORKSPACE,
                     "kv_write_attention_static: the plan needs " + std::to_string(need) +
                         " workspace bytes, more than the static scratch's " +
                         std::to_string(CPA_STATIC_SCRATCH_BYTES));
  if (!q || !k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !block_table || !out)
    return cpa::fail(CPA_ERR_INVALID_ARG, "kv_write_attention_static: NULL pointer");
  void* ws = nullptr;
  cpa_status st = cpa::scratch_on_current_device(&ws);
  if (st != CPA_OK) return st;
  if (!cpa::workspace_holds(plan, ws)) {
    st = cpa_plan_upload(plan, ws, CPA_STATIC_SCRATCH_BYTES, stream);
    if (st != CPA_OK) return st;
  }
  return cpa_kv_write_attention(plan, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                block_table, out, ws, CPA_STATIC_SCRATCH_BYTES, stream);
}
