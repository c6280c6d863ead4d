// api.cpp -- status strings and the optional kernel-timing recorder of the C ABI.
#include <hip/hip_runtime.h>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>
#include "../../include/ttt_lact.h"
#include "timing.hpp"

extern "C" const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_ARG: return "invalid argument (null pointer, negative size or bad enum)";
    case TTT_ERR_SHAPE: return "inconsistent or unsupported shape";
    case TTT_ERR_UNSUPPORTED: return "combination not implemented";
    case TTT_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TTT_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

namespace ttt {
namespace {
thread_local char last_error[512] = "";
}  // namespace

void note_hip_error(const char* what, hipError_t e, const char* file, int line) {
  const char* base = std::strrchr(file, '/');
  std::snprintf(last_error, sizeof last_error, "%s (%s) at %s:%d: %s", hipGetErrorName(e), hipGetErrorString(e),
                base ? base + 1 : file, line, what);
}

void note_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(last_error, sizeof last_error, fmt, ap);
  va_end(ap);
}
}  // namespace ttt

extern "C" const char* ttt_last_error(void) { return ttt::last_error; }

namespace ttt {
namespace {
const char* kClassNames[K_NUM_CLASSES] = {
    "lact_init", "lact_grad", "lact_update", "lact_apply", "lact_final",
    "linattn_prep", "linattn_delta", "linattn_scan", "linattn_apply", "linattn_fused",
    "inplace_prep", "inplace_z", "inplace_apply", "inplace_update", "lact_update_apply",
    "inplace_apply_z", "inplace_swiglu_bwd", "inplace_wgrad"};
struct Rec { int cls; hipEvent_t a, b; };
std::mutex mu;
bool on = false;
std::vector<Rec> recs;
std::vector<hipEvent_t> pool;  // events not in use
}  // namespace

bool timing_on() { return on; }

hipEvent_t timing_event() {
  std::lock_guard<std::mutex> g(mu);
  if (!pool.empty()) {
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timing_record(int cls, hipEvent_t a, hipEvent_t b) {
  std::lock_guard<std::mutex> g(mu);
  recs.push_back({cls, a, b});
}
}  // namespace ttt

extern "C" ttt_status ttt_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> g(ttt::mu);
  ttt::on = enable != 0;
  if (!ttt::on && ttt::recs.empty()) {
    // release the pooled events while the runtime is alive (none is left for process teardown)
    ttt_status st = TTT_OK;
    for (hipEvent_t e : ttt::pool)
      if (hipEventDestroy(e) != hipSuccess) st = TTT_ERR_HIP;
    ttt::pool.clear();
    return st;
  }
  return TTT_OK;
}

extern "C" ttt_status ttt_timing_collect(ttt_kernel_time* out, int32_t capacity, int32_t* count) {
  using namespace ttt;
  std::vector<Rec> rs;
  {
    std::lock_guard<std::mutex> g(mu);
    rs.swap(recs);
  }
  int launches[K_NUM_CLASSES] = {0};
  float ms[K_NUM_CLASSES] = {0.f};
  ttt_status st = TTT_OK;
  for (const Rec& r : rs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) st = TTT_ERR_HIP;
    launches[r.cls] += 1;
    ms[r.cls] += t;
  }
  {
    std::lock_guard<std::mutex> g(mu);
    for (const Rec& r : rs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
  }
  int n = 0;
  for (int c = 0; c < K_NUM_CLASSES; ++c) {
    if (!launches[c]) continue;
    if (out && n < capacity) out[n] = ttt_kernel_time{kClassNames[c], launches[c], ms[c]};
    ++n;
  }
  if (count) *count = n;
  return st;
}

// the parameter structs' layouts are part of the ABI (the Python binding mirrors them)
static_assert(sizeof(ttt_lact_params) == 88, "ttt_lact_params layout");
static_assert(sizeof(ttt_linattn_params) == 56, "ttt_linattn_params layout");
static_assert(sizeof(ttt_inplace_params) == 72, "ttt_inplace_params layout");
