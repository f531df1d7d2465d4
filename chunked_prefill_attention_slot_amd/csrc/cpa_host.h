// Host-side helpers shared by the C ABI translation units: the per-thread
// error message behind cpa_last_error().
#pragma once

#include <string>

#include "cpa.h"

namespace cpa {

std::string& last_error();

// Device workspace bytes `plan` needs (0 for a NULL plan).
size_t plan_workspace_bytes(cpa_plan plan);
// Whether `workspace` holds `plan`'s work lists (its last cpa_plan_upload).
bool workspace_holds(cpa_plan plan, const void* workspace);

inline cpa_status fail(cpa_status code, const std::string& msg) {
  last_error() = msg;
  return code;
}

inline cpa_status ok() {
  last_error().clear();
  return CPA_OK;
}

}  // namespace cpa
