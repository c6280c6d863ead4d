// host.hpp -- host-side helpers shared by the entry points (validation, workspace planning).
#pragma once
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cfloat>
#include <cstddef>
#include <cstdint>
#include "../../include/ttt_lact.h"

namespace ttt {

// Records the failing HIP call for ttt_last_error() (per host thread).
void note_hip_error(const char* what, hipError_t e, const char* file, int line);
// Records a printf-style message for ttt_last_error() (per host thread).
void note_error(const char* fmt, ...);

#define TTT_HIP(expr)                                        \
  do {                                                       \
    hipError_t _e = (expr);                                  \
    if (_e != hipSuccess) {                                  \
      ::ttt::note_hip_error(#expr, _e, __FILE__, __LINE__);  \
      return TTT_ERR_HIP;                                    \
    }                                                        \
  } while (0)

// Sub-allocations of the caller's workspace, each 256-byte aligned.
struct WorkspacePlan {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t off = total;
    total += (bytes + 255) & ~size_t(255);
    return off;
  }
};

// Raise a kernel's dynamic-LDS limit once per instantiation.
template <class F>
inline hipError_t allow_lds(F* kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace ttt
