// Stand-ins for the GPU side of libcpa in the host sanitizer build: the
// kernel launchers and the two HIP runtime calls the host code makes. Every
// one reports that there is no device, so an entry point that would queue
// GPU work returns CPA_ERR_HIP instead; the planner, validator, predictor,
// calibration, scheduler and split point run exactly as in the product.
#include <hip/hip_runtime_api.h>

#include "cpa.h"
#include "cpa_host.h"
#include "cpa_internal.h"

namespace cpa {

hipError_t launch_prefill(const WorkItem*, int, const AttnArgs&, int, bool, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode(const WorkItem*, int, const AttnArgs&, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_combine(const CombineItem*, int, int, int, const AttnArgs&, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_kv_write(const uint16_t*, const uint16_t*, const int32_t*, int32_t, uint16_t*,
                           uint16_t*, int32_t, int32_t, int32_t, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace cpa

extern "C" {

const char* hipGetErrorString(hipError_t) { return "no device (host sanitizer build)"; }

#ifdef CPA_STUB_COPY_OK
// ThreadSanitizer build: a plan upload "succeeds" without touching the
// workspace, so the uploads of many threads reach the workspace registry.
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipSuccess;
}
#else
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNoDevice;
}
#endif

cpa_status cpa_kv_write_attention_static(cpa_plan, const void*, const void*, const void*,
                                         const int32_t*, void*, void*, const int32_t*, void*,
                                         hipStream_t) {
  return cpa::fail(CPA_ERR_UNSUPPORTED, "host sanitizer build: no device");
}

}  // extern "C"
