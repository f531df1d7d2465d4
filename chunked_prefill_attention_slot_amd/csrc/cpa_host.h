// Host-side helpers shared by the C ABI translation units: the per-thread
// error message behind cpa_last_error().
#pragma once

#include <string>

#include "cpa.h"

namespace cpa {

std::string& last_error();

inline cpa_status fail(cpa_status code, const std::string& msg) {
  last_error() = msg;
  return code;
}

inline cpa_status ok() {
  last_error().clear();
  return CPA_OK;
}

}  // namespace cpa
