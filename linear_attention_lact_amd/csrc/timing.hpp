// timing.hpp -- optional per-kernel-class launch timing with HIP events (ttt_timing_*).
#pragma once
#include <hip/hip_runtime.h>

namespace ttt {

enum KernelClass {
  K_LACT_INIT = 0, K_LACT_GRAD, K_LACT_UPDATE, K_LACT_APPLY, K_LACT_FINAL,
  K_LIN_PREP, K_LIN_DELTA, K_LIN_SCAN, K_LIN_APPLY, K_LIN_FUSED,
  K_INP_PREP, K_INP_Z, K_INP_APPLY, K_INP_UPDATE,
  K_LACT_UPD_APPLY,  // weight update and the chunk's apply in one launch
  K_NUM_CLASSES
};

bool timing_on();
void timing_record(int cls, hipEvent_t a, hipEvent_t b);
hipEvent_t timing_event();

// Brackets the launches issued in its scope on `stream` when timing is enabled.
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

}  // namespace ttt
