// linattn.hip -- the last-layer-only linear-attention form on gfx950 (ttt_linattn_forward).
//
// With only W1 written and no renormalisation, the fast weight's kernel
// phi(x) = silu(x W0) * (x W2) is static and the state update is associative (KV-binding
// summary page, "Prerequisites -> Linear attention" and Theorem 5.2 under "Method step
// details"; press article, section 4). Per pair:
//   dS_c = phi(K_c)^T diag(eta_c) V_c                    (grad_kernel, linear-attention mode)
//   S_c  = W1 + sum_{j<c} dS_j   (apply-then-update)  or  sum_{j<=c} (update-then-apply)
//          (with momentum, each dS_j weighted by its cumulative coefficient, Theorem 5.3)
//   O_c  = phi(Q_c) S_c                                   (apply_kernel with per-chunk S_c)
// The chunk prefix is an exclusive (or inclusive) scan over the chunks of each pair.
#include <cstdlib>
#include <mutex>

#include "fastweight.hpp"
#include "linattn_fused.hpp"
#include "linattn_scan.hpp"
#include "host.hpp"
#include "timing.hpp"

namespace ttt {

template <class IoT, class OpT, int H>
static ttt_status linattn_run(const ttt_linattn_params& p, char* ws, size_t oSh, size_t odS, size_t oSt,
                              const void* Q, const void* K, const void* V, const float* eta,
                              const float* W0, const float* W2, const float* W1, void* O, float* S_out,
                              hipStream_t st) {
  constexpr bool RD = H <= 128;  // register-direct chunk-aggregate kernel
  auto gk = grad_kernel<IoT, OpT, H, true, false>;
  auto gkr = grad_rd_kernel<IoT, OpT, (RD ? H : 128), true, false>;
  auto ak = apply_kernel<IoT, OpT, H>;
  // register-direct apply where its double-buffered weight blocks fit in LDS
  constexpr bool ARD = H <= 128 && apply_rd_lds_bytes<OpT, (H <= 128 ? H : 128)>() <= 160 * 1024;
  auto akr = apply_rd_kernel<IoT, OpT, (ARD ? H : 64)>;
  constexpr int glds = RD ? grad_rd_lds_bytes<OpT, (RD ? H : 128), true>() : grad_lds_bytes<OpT, H, true>();
  constexpr int alds = ARD ? apply_rd_lds_bytes<OpT, (ARD ? H : 64)>() : apply_lds_bytes<OpT, H>();
  static_assert(glds <= 160 * 1024 && alds <= 160 * 1024, "LDS budget");
  static const hipError_t lds_ok = [&] {
    hipError_t e = RD ? allow_lds(gkr, glds) : allow_lds(gk, glds);
    return e != hipSuccess ? e : (ARD ? allow_lds(akr, alds) : allow_lds(ak, alds));
  }();
  TTT_HIP(lds_ok);
  const int P = p.B * p.H, rh = p.r * H, nch = p.N / p.chunk;
  const int64_t n = (int64_t)rh * H;
  OpT* sh = reinterpret_cast<OpT*>(ws + oSh);
  float* dS = reinterpret_cast<float*>(ws + odS);
  OpT* St = reinterpret_cast<OpT*>(ws + oSt);

  {
    LaunchTimer lt(K_LIN_PREP, st);
    hipLaunchKernelGGL(linattn_prep_kernel<OpT>, dim3((unsigned)((rh / 32) * (H / 32)), 2, P), dim3(256), 0, st,
                       W0, W2, sh, p.H, H, rh, p.w_batch_stride);
    TTT_HIP(hipGetLastError());
  }
  GradArgs ga{};
  ga.K = K;
  ga.V = V;
  ga.eta = eta;
  ga.tok_pair_stride = (int64_t)p.N * H;
  ga.eta_pair_stride = p.N;
  ga.t_base = 0;
  ga.seg_len = p.chunk;
  ga.t_limit = p.N;
  ga.W0T = sh;
  ga.W2T = sh + n;
  ga.W1 = nullptr;
  ga.w_pair_stride = 2 * n;
  ga.rh = rh;
  ga.out = dS;
  ga.out_y_stride = n;
  ga.out_pair_stride = (int64_t)nch * n;
  ga.out_mat_stride = 0;
  {
    LaunchTimer lt(K_LIN_DELTA, st);
    if constexpr (RD) {
      const unsigned grid = (unsigned)(rh / RB) * 8u * (unsigned)((P * nch + 7) / 8);
      hipLaunchKernelGGL(gkr, dim3(grid), dim3(256), glds, st, ga, nch, P);
    } else {
      hipLaunchKernelGGL(gk, dim3(rh / RB, nch, P), dim3(256), glds, st, ga);
    }
    TTT_HIP(hipGetLastError());
  }
  {
    LaunchTimer lt(K_LIN_SCAN, st);
    auto sk = linattn_scan_kernel<OpT, ARD>;
    hipLaunchKernelGGL(sk, dim3((unsigned)((n + 255) / 256), P), dim3(256), 0, st, W1, dS,
                       St, S_out, p.H, H, rh, nch, p.order == TTT_UPDATE_THEN_APPLY ? 1 : 0, p.momentum,
                       p.w_batch_stride, p.chunk_flags);
    TTT_HIP(hipGetLastError());
  }
  ApplyArgs aa{};
  aa.Q = Q;
  aa.tok_pair_stride = (int64_t)p.N * H;
  aa.t_base = 0;
  aa.t_limit = p.N;
  aa.tiles_per_chunk = ARD ? (p.chunk + AT - 1) / AT : (p.chunk + TT - 1) / TT;
  aa.W0T = sh;
  aa.W2T = sh + n;
  aa.w_pair_stride = 2 * n;
  aa.W1T = St;
  aa.w1t_pair_stride = (int64_t)nch * n;
  aa.w1t_chunk_stride = n;
  aa.W1 = St;
  aa.w1_pair_stride = (int64_t)nch * n;
  aa.w1_chunk_stride = n;
  aa.chunk = p.chunk;
  aa.rh = rh;
  aa.O = O;
  aa.npairs = P;
  aa.ntiles = nch * aa.tiles_per_chunk;
  {
    LaunchTimer lt(K_LIN_APPLY, st);
    const dim3 agrid(8u * (unsigned)((P + 7) / 8) * (unsigned)aa.ntiles);
    if constexpr (ARD)
      hipLaunchKernelGGL(akr, agrid, dim3(512), alds, st, aa);
    else
      hipLaunchKernelGGL(ak, agrid, dim3(256), alds, st, aa);
    TTT_HIP(hipGetLastError());
  }
  return TTT_OK;
}

// Single-pass path (linattn_fused.hpp) for rh <= 128.
template <class IoT, class OpT, int H, int RH, bool MOM, bool ID = false>
static ttt_status linattn_fused_run(const ttt_linattn_params& p, char* ws, size_t oAgg, size_t oIncl, size_t oInclM,
                                    size_t oFl, size_t oTk, const void* Q, const void* K, const void* V,
                                    const float* eta, const float* W0, const float* W2, const float* W1, void* O,
                                    float* S_out, hipStream_t st) {
  typedef FusedLayout<OpT, H, RH, ID> FL;
  auto fk = linattn_fused_kernel<IoT, OpT, H, RH, MOM, ID>;
  constexpr int lds = linattn_fused_lds_bytes<OpT, H, RH, ID>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t lds_ok = allow_lds(fk, lds);
  TTT_HIP(lds_ok);
  const int P = p.B * p.H, nch = p.N / p.chunk;
  FusedArgs fa{};
  fa.Q = Q;
  fa.K = K;
  fa.V = V;
  fa.eta = eta;
  fa.W0 = W0;
  fa.W2 = W2;
  fa.W1 = W1;
  fa.O = O;
  fa.S_out = S_out;
  fa.agg = reinterpret_cast<float*>(ws + oAgg);
  fa.incl = reinterpret_cast<float*>(ws + oIncl);
  fa.inclm = MOM ? reinterpret_cast<float*>(ws + oInclM) : nullptr;
  fa.alpha = p.momentum;
  fa.flags = reinterpret_cast<unsigned*>(ws + oFl);
  fa.tickets = reinterpret_cast<unsigned*>(ws + oTk);
  fa.P = P;
  fa.heads = p.H;
  fa.N = p.N;
  fa.chunk = p.chunk;
  fa.nch = nch;
  fa.inclusive = p.order == TTT_UPDATE_THEN_APPLY ? 1 : 0;
  fa.w_batch_stride = p.w_batch_stride;
  // chunks per workgroup: the workgroups hold one CU each (LDS), so groups of G chunks bring the
  // grid down to one round over the device's CUs where the chunk splits into whole query passes
  constexpr int PASS = FL::NW * 32;
  constexpr int GLIM = MOM ? FL::GMAX : 8;  // the momentum lookback holds up to GMAX partial sums
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || ncu <= 0)
    return TTT_ERR_HIP;
  int G = 1;
  while (G < GLIM && (int64_t)8 * ((P + 7) / 8) * (nch / G) > ncu && nch % (2 * G) == 0 && p.chunk % PASS == 0)
    G *= 2;
  fa.group = G;
  {  // test hook: the lookback stress seed (see linattn_fused.hpp)
    const char* sv = std::getenv("TTT_LOOKBACK_STRESS");
    fa.stress = sv ? (unsigned)std::strtoul(sv, nullptr, 10) : 0u;
  }
  {
    LaunchTimer lt(K_LIN_PREP, st);
    hipLaunchKernelGGL(linattn_fused_reset, dim3(1), dim3(256), 0, st, fa.tickets, fa.flags, P * nch);
    TTT_HIP(hipGetLastError());
  }
  const unsigned grid = 8u * (unsigned)((P + 7) / 8) * (unsigned)(nch / G);
  TTT_HIP(launch_k(K_LIN_FUSED, fk, dim3(grid), dim3(FL::NT), lds, st, fa));
  return TTT_OK;
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_linattn_forward(const ttt_linattn_params* p, const void* Q, const void* K,
                                          const void* V, const float* eta, const float* W0,
                                          const float* W2, const float* W1, void* O, float* S_out,
                                          void* workspace, size_t* workspace_bytes, void* stream) {
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_linattn_params& q = *p;
  if (q.B < 0 || q.H < 0 || q.N < 0 || q.h <= 0 || q.r <= 0 || q.chunk <= 0) return TTT_ERR_ARG;
  if (q.order != TTT_APPLY_THEN_UPDATE && q.order != TTT_UPDATE_THEN_APPLY) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (q.w_batch_stride < 0) return TTT_ERR_ARG;
  if (!(q.momentum >= 0.f && q.momentum < 1.f)) return TTT_ERR_ARG;  // also rejects NaN
  if (q.feature_map != TTT_PHI_SWIGLU && q.feature_map != TTT_PHI_IDENTITY) return TTT_ERR_ARG;
  const bool ident = q.feature_map == TTT_PHI_IDENTITY;
  if (ident && q.r != 1) return TTT_ERR_ARG;  // the identity map's state is h x h
  if (q.N % q.chunk) return TTT_ERR_SHAPE;
  const int64_t rh64 = (int64_t)q.r * q.h;
  if (q.h % 32 || (!ident && rh64 % 64) || rh64 > 1024) return TTT_ERR_SHAPE;
  if (q.w_batch_stride != 0 && q.w_batch_stride != (int64_t)q.H * rh64 * q.h) return TTT_ERR_SHAPE;
  const bool bf16 = q.dtype == TTT_BF16;
  if (bf16 ? (q.h > 256) : (q.h > 128)) return TTT_ERR_UNSUPPORTED;
  const int P = q.B * q.H, nch = q.N / q.chunk;
  if (P > 0 && (!W1 || (!ident && (!W0 || !W2)))) return TTT_ERR_ARG;
  if (P > 0 && nch > 0 && (!Q || !K || !V || !eta || !O)) return TTT_ERR_ARG;
  const int64_t n = rh64 * q.h;
  const size_t opsz = bf16 ? 2 : 4;
  // single pass for bf16 I/O and (h, rh) in {(32, 64), (32, 128), (64, 128)}
  // the single-pass kernel keeps each pair's chunks on one XCD (its L2 is where the chunks
  // exchange their sums): it needs a device of 8 XCDs, which dispatches workgroups to them in turn
  int dev = 0, nxcc = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&nxcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess)
    nxcc = 0;
  // the identity map: single pass only, h in {64, 128}
  const bool shape_ok = ident ? (q.h == 64 || q.h == 128)
                              : ((q.h == 32 && (rh64 == 64 || rh64 == 128)) || (q.h == 64 && rh64 == 128));
  const bool fused_shape = bf16 && shape_ok &&
                           (int64_t)nch * rh64 * q.h * 4 < (int64_t)1 << 31 &&  // buffer offsets are 32-bit
                           (int64_t)q.N * q.h * 2 < (int64_t)1 << 31;
  // per-chunk flags run on the multi-launch path (its scan walks the chunks one by one); the
  // identity map has no such path
  const bool flagged = q.chunk_flags != nullptr;
  if (ident && (flagged || !fused_shape)) return TTT_ERR_UNSUPPORTED;
  const bool fused = fused_shape && nxcc == 8 && !flagged;
  // both plans; the size asked for covers the larger where the single-pass shape applies, so a
  // query gives the same answer on any device (and without one)
  WorkspacePlan fplan, mplan;
  const bool mom = q.momentum != 0.f;
  const size_t oAgg = fplan.add((size_t)P * nch * n * 4);
  const size_t oIncl = fplan.add((size_t)P * nch * n * 4);
  const size_t oInclM = mom ? fplan.add((size_t)P * nch * n * 4) : 0;
  const size_t oFl = fplan.add((size_t)P * nch * 4);
  const size_t oTk = fplan.add(16 * 4);
  const size_t oSh = mplan.add((size_t)P * 2 * n * opsz);
  const size_t odS = mplan.add((size_t)P * nch * n * 4);
  const size_t oSt = mplan.add((size_t)P * nch * n * opsz);
  const size_t need = ident ? fplan.total : (fused_shape && !flagged) ? std::max(fplan.total, mplan.total) : mplan.total;
  if (!workspace) {
    *workspace_bytes = need;
    return TTT_OK;
  }
  if (*workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (P == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (nch == 0) {  // empty sequences: the final state is W1
    if (S_out) {
      for (int b = 0; b < q.B; ++b)
        TTT_HIP(hipMemcpyAsync(S_out + (int64_t)b * q.H * n, W1 + (int64_t)b * q.w_batch_stride,
                               (size_t)q.H * n * 4, hipMemcpyDeviceToDevice, st));
    }
    return TTT_OK;
  }
  char* ws = static_cast<char*>(workspace);
  if (ident && !fused) {
    note_error("ttt_linattn_forward: the identity feature map runs on the single-pass path only, which "
               "needs a device with 8 XCDs");
    return TTT_ERR_UNSUPPORTED;
  }
  if (fused) {
    try {
#define TTT_FUSED(IOT, OPT, HH, RR)                                                                         \
  if (q.h == HH && rh64 == RR)                                                                              \
    return mom ? linattn_fused_run<IOT, OPT, HH, RR, true>(q, ws, oAgg, oIncl, oInclM, oFl, oTk, Q, K, V, eta, \
                                                           W0, W2, W1, O, S_out, st)                        \
               : linattn_fused_run<IOT, OPT, HH, RR, false>(q, ws, oAgg, oIncl, oInclM, oFl, oTk, Q, K, V,  \
                                                            eta, W0, W2, W1, O, S_out, st);
      if (ident) {
        if (q.h == 64)
          return mom ? linattn_fused_run<bf16_t, _Float16, 64, 64, true, true>(q, ws, oAgg, oIncl, oInclM, oFl, oTk,
                                                                               Q, K, V, eta, W0, W2, W1, O, S_out, st)
                     : linattn_fused_run<bf16_t, _Float16, 64, 64, false, true>(q, ws, oAgg, oIncl, oInclM, oFl, oTk,
                                                                                Q, K, V, eta, W0, W2, W1, O, S_out, st);
        if (q.h == 128)
          return mom ? linattn_fused_run<bf16_t, _Float16, 128, 128, true, true>(q, ws, oAgg, oIncl, oInclM, oFl, oTk,
                                                                                 Q, K, V, eta, W0, W2, W1, O, S_out, st)
                     : linattn_fused_run<bf16_t, _Float16, 128, 128, false, true>(q, ws, oAgg, oIncl, oInclM, oFl,
                                                                                  oTk, Q, K, V, eta, W0, W2, W1, O,
                                                                                  S_out, st);
        return TTT_ERR_UNSUPPORTED;
      }
      TTT_FUSED(bf16_t, _Float16, 32, 64)
      TTT_FUSED(bf16_t, _Float16, 32, 128)
      TTT_FUSED(bf16_t, _Float16, 64, 128)
#undef TTT_FUSED
    } catch (...) {
      return TTT_ERR_HIP;
    }
    return TTT_ERR_UNSUPPORTED;
  }
#define TTT_LIN_CASE(IOT, OPT, HH) \
  case HH:                         \
    return linattn_run<IOT, OPT, HH>(q, ws, oSh, odS, oSt, Q, K, V, eta, W0, W2, W1, O, S_out, st);
  try {
    if (bf16) {
      switch (q.h) {
        TTT_LIN_CASE(bf16_t, __bf16, 32)
        TTT_LIN_CASE(bf16_t, __bf16, 64)
        TTT_LIN_CASE(bf16_t, __bf16, 96)
        TTT_LIN_CASE(bf16_t, __bf16, 128)
        TTT_LIN_CASE(bf16_t, __bf16, 160)
        TTT_LIN_CASE(bf16_t, __bf16, 192)
        TTT_LIN_CASE(bf16_t, __bf16, 224)
        TTT_LIN_CASE(bf16_t, __bf16, 256)
        default: return TTT_ERR_UNSUPPORTED;
      }
    } else {
      switch (q.h) {
        TTT_LIN_CASE(float, float, 32)
        TTT_LIN_CASE(float, float, 64)
        TTT_LIN_CASE(float, float, 96)
        TTT_LIN_CASE(float, float, 128)
        default: return TTT_ERR_UNSUPPORTED;
      }
    }
  } catch (...) {
    return TTT_ERR_HIP;
  }
#undef TTT_LIN_CASE
}

// ---------------------------------------------------------------------------------------
// Allocation-free variant: the workspace is a file-scope device array of fixed size, one copy
// per GPU the library runs on (held until the process ends). Its device address is looked up
// once per device with that device current; host code uses only that address.
namespace ttt {
namespace {
__device__ __align__(256) unsigned char noalloc_scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return hipSuccess;
}
}  // namespace
}  // namespace ttt

extern "C" ttt_status ttt_linattn_forward_noalloc(const ttt_linattn_params* p, const void* Q, const void* K,
                                                  const void* V, const float* eta, const float* W0,
                                                  const float* W2, const float* W1, void* O, float* S_out,
                                                  void* stream) {
  size_t need = 0;
  const ttt_status q = ttt_linattn_forward(p, Q, K, V, eta, W0, W2, W1, O, S_out, nullptr, &need, stream);
  if (q != TTT_OK) return q;
  if (need > (size_t)TTT_NOALLOC_SCRATCH_BYTES) {
    note_error("ttt_linattn_forward_noalloc: the call needs %zu bytes of scratch, more than the %zu the "
               "library holds per device; use ttt_linattn_forward with a workspace",
               need, (size_t)TTT_NOALLOC_SCRATCH_BYTES);
    return TTT_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  TTT_HIP(noalloc_scratch_ptr(&ws));
  size_t have = TTT_NOALLOC_SCRATCH_BYTES;
  return ttt_linattn_forward(p, Q, K, V, eta, W0, W2, W1, O, S_out, ws, &have, stream);
}
