// Host-side helpers shared by the ABI translation units.  Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"

namespace bgtq {

bgtq_status fail(bgtq_status s, const std::string &m);
bgtq_status launch_status(const char *what);
int device_cus();

// Events bracketing the cache-streaming kernel while profiling is on.
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending, pool;
};
Prof &prof();

}  // namespace bgtq
