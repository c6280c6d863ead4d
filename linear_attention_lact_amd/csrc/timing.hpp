// timing.hpp -- optional per-kernel-class launch timing with HIP events (ttt_timing_*).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>

namespace ttt {

enum KernelClass {
  K_LACT_INIT = 0, K_LACT_GRAD, K_LACT_UPDATE, K_LACT_APPLY, K_LACT_FINAL,
  K_LIN_PREP, K_LIN_DELTA, K_LIN_SCAN, K_LIN_APPLY, K_LIN_FUSED,
  K_INP_PREP, K_INP_Z, K_INP_APPLY, K_INP_UPDATE,
  K_LACT_UPD_APPLY,  // weight update and the chunk's apply in one launch
  K_INP_APPLY_Z,     // In-Place apply of a chunk and the next chunk's Z in one launch
  K_INP_SWIGLU_BWD,  // In-Place backward: dZ with the SwiGLU-backward epilogue
  K_INP_WGRAD,       // In-Place backward: the gate and up projections' gradients over a sequence
  K_NUM_CLASSES
};

bool timing_on();
void timing_record(int cls, hipEvent_t a, hipEvent_t b);
hipEvent_t timing_event();

// Brackets the launches issued in its scope on `stream` when timing is enabled (events recorded
// on the stream before and after: the span includes the dispatch of the first launch).
struct LaunchTimer {
  int cls;
  hipStream_t st;
  hipEvent_t a = nullptr;
  LaunchTimer(int c, hipStream_t s) : cls(c), st(s) {
    if (timing_on()) {
      a = timing_event();
      if (a) (void)hipEventRecord(a, st);
    }
  }
  ~LaunchTimer() {
    if (a) {
      hipEvent_t b = timing_event();
      if (b) {
        (void)hipEventRecord(b, st);
        timing_record(cls, a, b);
      }
    }
  }
};

// One kernel launch; when timing is enabled the start and stop events are attached to the
// dispatch itself (hipExtLaunchKernel), so they carry the kernel's own begin and end timestamps,
// the figures a kernel trace reports.
inline hipError_t launch_raw(int cls, const void* f, dim3 grid, dim3 block, void** args, size_t lds, hipStream_t st) {
  hipEvent_t a = timing_on() ? timing_event() : nullptr;
  hipEvent_t b = a ? timing_event() : nullptr;
  if (a && b) {
    const hipError_t e = hipExtLaunchKernel(f, grid, block, args, lds, st, a, b, 0);
    if (e == hipSuccess) timing_record(cls, a, b);
    return e;
  }
  const hipError_t e = hipLaunchKernel(f, grid, block, args, lds, st);
  return e != hipSuccess ? e : hipGetLastError();
}

template <typename... KArgs, typename... Args>
inline hipError_t launch_k(int cls, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                           Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  std::tuple<KArgs...> t{static_cast<KArgs>(args)...};
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... x) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&x)), ...);
  }, t);
  return launch_raw(cls, reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, st);
}

}  // namespace ttt
