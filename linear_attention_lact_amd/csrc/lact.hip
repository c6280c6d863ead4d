// lact.hip -- the chunked LaCT fast-weight layer on gfx950 (ttt_lact_forward).
//
// Per (sequence, head) pair and chunk (sources: KV-binding summary page, "Prerequisites ->
// LaCT"; "Test-Time Training Done Right" reading notes, sections 2.1-2.3; "In-Place
// Test-Time Training" notes, section 3.1):
//   apply: O_c = (silu(Q_c W0) * (Q_c W2)) W1
//   write: G = gradients of -sum eta <f(k), v> at the chunk-start weights (grad_kernel),
//          U = G, or M = momentum*M + G and U = M; optionally U = NS5(U); W -= U;
//          optionally each output column renormalised over its inputs to its initial norm.
// Launch sequence per chunk: [apply] -> grad -> update -> [apply], all on the caller's stream.
//
// State layout in the workspace (float32, per pair): W0T [rh][h], W1 [rh][h], W2T [rh][h];
// the same for the momentum buffers. Row j of W0T / W2T is input-weight column j of W0 / W2,
// so the renormalisation of W0 / W2 is a row norm here and that of W1 a column norm.
#include "fastweight.hpp"
#include "host.hpp"
#include "timing.hpp"
#include "update.hpp"
#include "update_tiled.hpp"

namespace ttt {

// ---------------------------------------------------------------------------------------
// init: the initial state (W0, W2 transposed into rows of hidden units), momentum and both
// operand shadow buffers (a matrix outside the update mask keeps its initial shadow in each).
// grid (rh/32 * h/32, 3, P), block 256: one 32 x 32 tile of the state (rows j, columns c);
// W0/W2 and their momentum arrive in row form [h][rh] and are transposed through LDS.
template <class OpT>
__global__ void __launch_bounds__(256) lact_init_kernel(LactState s, const float* W0, const float* W1,
                                                       const float* W2, const float* M_in, int H,
                                                       int64_t w_batch_stride) {
  __shared__ float tw[32][33], tm[32][33];
  const int mat = blockIdx.y, pair = blockIdx.z;
  const int h = s.h, rh = s.rh, hb = h / 32;
  const int64_t n = (int64_t)rh * h;
  const int j0 = (blockIdx.x / hb) * 32, c0 = (blockIdx.x % hb) * 32;
  const int b = pair / H, head = pair % H;
  const float* src = (mat == 0 ? W0 : mat == 1 ? W1 : W2) + (int64_t)b * w_batch_stride + (int64_t)head * n;
  const float* msrc = M_in ? M_in + ((int64_t)pair * 3 + mat) * n : nullptr;
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  // row-form tile rows: state rows j (W1) or input columns c (W0, W2)
  const int64_t so = mat == 1 ? (int64_t)(j0 + r) * h + c0 + c4 : (int64_t)(c0 + r) * rh + j0 + c4;
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + so);
  const f32x4 m = msrc ? *reinterpret_cast<const f32x4*>(msrc + so) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    tw[r][c4 + q] = v[q];
    tm[r][c4 + q] = m[q];
  }
  __syncthreads();
  f32x4 sv = v, sm = m;  // state row j0 + r, columns c0 + c4..
  if (mat != 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sv[q] = tw[c4 + q][r];
      sm[q] = tm[c4 + q][r];
    }
  }
  const int64_t e = (int64_t)(j0 + r) * h + c0 + c4;
  *reinterpret_cast<f32x4*>(s.W + ((int64_t)pair * 3 + mat) * n + e) = sv;
  *reinterpret_cast<f32x4*>(s.M + ((int64_t)pair * 3 + mat) * n + e) = sm;
  for (int buf = 0; buf < 2; ++buf) {
    OpT* sh = reinterpret_cast<OpT*>(s.sh) + ((int64_t)buf * s.P + pair) * 4 * n;
    OpT* d = sh + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n + e;
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = Mfma<OpT>::from_f32(sv[q]);
    if (mat == 1) {  // W1^T [h][rh]: row c0 + r, columns j0 + c4..
      OpT* dt = sh + 3 * n + (int64_t)(c0 + r) * rh + j0 + c4;
#pragma unroll
      for (int q = 0; q < 4; ++q) dt[q] = Mfma<OpT>::from_f32(tw[c4 + q][r]);
    }
  }
}

// The weight update of chunk c and the apply of the same chunk (apply-then-update order) in
// one launch: the first nupd workgroups run the update (one matrix each, writing the other
// shadow buffer), the rest the apply (reading the shadows the chunk's gradient used). The
// update occupies one CU per matrix; the apply's workgroups fill the remaining CUs meanwhile.
template <class IoT, class OpT, int H, int RH>
__global__ void __launch_bounds__(512) lact_update_apply_kernel(UpdateArgs u, ApplyArgs a, int nupd) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < nupd)
    lact_update_body<OpT, H, RH>(u, blockIdx.x, smem);
  else
    apply_rd_body<IoT, OpT, H>(a, blockIdx.x - nupd, smem);
}

// renorm targets (column norms of the initial row-form weights over their input axis).
// grid (3, P), block 256; the row loop is unrolled so that eight loads are in flight.
__global__ void __launch_bounds__(256) lact_norms_kernel(LactState s, const float* W0, const float* W1,
                                                        const float* W2, int H, int64_t w_batch_stride) {
  const int mat = blockIdx.x, pair = blockIdx.y;
  const int h = s.h, rh = s.rh;
  const int64_t n = (int64_t)rh * h;
  const int b = pair / H, head = pair % H;
  const float* src = (mat == 0 ? W0 : mat == 1 ? W1 : W2) + (int64_t)b * w_batch_stride + (int64_t)head * n;
  float* nu = s.nu + ((int64_t)pair * 3 + mat) * s.NU;
  const int cols = mat == 1 ? h : rh, rows = mat == 1 ? rh : h;  // row-form [rows][cols]
  for (int j = threadIdx.x; j < cols; j += 256) {
    float acc = 0.f;
#pragma unroll 8
    for (int r = 0; r < rows; ++r) acc += src[(int64_t)r * cols + j] * src[(int64_t)r * cols + j];
    nu[j] = sqrtf(acc);
  }
}

// power-of-two step-size scales of the gradient's token segments: for chunk c, pair p and
// segment g, 2^-floor(log2(max eta)) over the segment's tokens (1 when the maximum is 0).
// grid (P, nch), block 256; out [nch][P][S].
__global__ void __launch_bounds__(256) lact_eta_scale_kernel(const float* eta, int64_t eta_pair_stride, int chunk,
                                                            int seg_len, int S, float* out) {
  __shared__ float red[16];
  const int pair = blockIdx.x, c = blockIdx.y, P = gridDim.x;
  const float* ep = eta + pair * eta_pair_stride;
  for (int g = 0; g < S; ++g) {
    const int t0 = c * chunk + g * seg_len, t1 = min(t0 + seg_len, (c + 1) * chunk);
    float mx = 0.f;
    for (int t = t0 + threadIdx.x; t < t1; t += 256) mx = fmaxf(mx, ep[t]);
    mx = block_max(mx, red);
    if (threadIdx.x == 0) out[((int64_t)c * P + pair) * S + g] = mx > 0.f ? exp2f(-floorf(log2f(mx))) : 1.f;
  }
}

// finalize: state and momentum back to the API's row form (W0/W2 transposed through LDS).
// grid (rh/32 * h/32, 3, P), block 256: one 32 x 32 state tile.
__global__ void __launch_bounds__(256) lact_final_kernel(LactState s, float* W0o, float* W1o, float* W2o,
                                                        float* Mo) {
  __shared__ float tw[32][33], tm[32][33];
  const int mat = blockIdx.y, pair = blockIdx.z;
  const int h = s.h, rh = s.rh, hb = h / 32;
  const int64_t n = (int64_t)rh * h;
  const int j0 = (blockIdx.x / hb) * 32, c0 = (blockIdx.x % hb) * 32;
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  const int64_t e = (int64_t)(j0 + r) * h + c0 + c4;
  f32x4 v = *reinterpret_cast<const f32x4*>(s.W + ((int64_t)pair * 3 + mat) * n + e);
  f32x4 m = *reinterpret_cast<const f32x4*>(s.M + ((int64_t)pair * 3 + mat) * n + e);
  int64_t d = e;  // row-form offset of this thread's four outputs
  if (mat != 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tw[r][c4 + q] = v[q];
      tm[r][c4 + q] = m[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = tw[c4 + q][r];
      m[q] = tm[c4 + q][r];
    }
    d = (int64_t)(c0 + r) * rh + j0 + c4;
  }
  float* wo = (mat == 0 ? W0o : mat == 1 ? W1o : W2o);
  if (wo) *reinterpret_cast<f32x4*>(wo + (int64_t)pair * n + d) = v;
  if (Mo) *reinterpret_cast<f32x4*>(Mo + ((int64_t)pair * 3 + mat) * n + d) = m;
}

// ---------------------------------------------------------------------------------------
template <class IoT, class OpT, int H>
static ttt_status lact_run(const ttt_lact_params& p, const LactState& s, int S, const void* Q,
                           const void* K, const void* V, const float* eta, const float* W0,
                           const float* W1, const float* W2, const float* M_in, void* O, float* W0o,
                           float* W1o, float* W2o, float* Mo, hipStream_t st) {
  constexpr bool SCALE = sizeof(OpT) == 2;
  constexpr bool RD = H <= 128;  // register-direct gradient kernel
  constexpr bool WS = std::is_same<OpT, _Float16>::value && (H == 64 || H == 128);  // its role-split form
  auto gk = grad_kernel<IoT, OpT, H, false, SCALE>;
  auto gkr = grad_rd_kernel<IoT, OpT, (RD ? H : 128), false, SCALE>;
  auto gkw = grad_ws_kernel<typename std::conditional<WS, IoT, bf16_t>::type, _Float16, (WS ? H : 128), true>;
  auto ak = apply_kernel<IoT, OpT, H>;
  // register-direct apply where its double-buffered weight blocks fit in LDS
  constexpr bool ARD = H <= 128 && apply_rd_lds_bytes<OpT, (H <= 128 ? H : 128)>() <= 160 * 1024;
  auto akr = apply_rd_kernel<IoT, OpT, (ARD ? H : 64)>;
  constexpr int glds = WS   ? grad_ws_lds_bytes<_Float16, (WS ? H : 128)>()
                       : RD ? grad_rd_lds_bytes<OpT, (RD ? H : 128), false>()
                            : grad_lds_bytes<OpT, H, false>();
  constexpr int alds = ARD ? apply_rd_lds_bytes<OpT, (ARD ? H : 64)>() : apply_lds_bytes<OpT, H>();
  static_assert(glds <= 160 * 1024 && alds <= 160 * 1024, "LDS budget");
  static const hipError_t lds_ok = [&] {
    hipError_t e = WS ? allow_lds(gkw, glds) : RD ? allow_lds(gkr, glds) : allow_lds(gk, glds);
    return e != hipSuccess ? e : (ARD ? allow_lds(akr, alds) : allow_lds(ak, alds));
  }();
  TTT_HIP(lds_ok);

  const int P = s.P, rh = s.rh;
  const int64_t n = (int64_t)rh * H;
  const int nch = p.Nk / p.chunk_kv;
  {
    LaunchTimer lt(K_LACT_INIT, st);
    hipLaunchKernelGGL(lact_init_kernel<OpT>, dim3((unsigned)(n / 1024), 3, P), dim3(256), 0, st, s, W0, W1,
                       W2, M_in, p.H, p.w_batch_stride);
    TTT_HIP(hipGetLastError());
    hipLaunchKernelGGL(lact_norms_kernel, dim3(3, P), dim3(256), 0, st, s, W0, W1, W2, p.H, p.w_batch_stride);
    TTT_HIP(hipGetLastError());
  }

  // operand shadows, double-buffered: chunk c's gradient and apply read buffer c & 1 while its
  // update writes buffer (c + 1) & 1
  const OpT* sh = reinterpret_cast<const OpT*>(s.sh);
  const int64_t shb = (int64_t)P * 4 * n;
  ApplyArgs aa{};
  aa.Q = Q;
  aa.tok_pair_stride = (int64_t)p.Nq * H;
  aa.W0T = sh;
  aa.W2T = sh + n;
  aa.w_pair_stride = 4 * n;
  aa.W1T = sh + 3 * n;
  aa.w1t_pair_stride = 4 * n;
  aa.w1t_chunk_stride = 0;
  aa.chunk = p.chunk_q;
  aa.tiles_per_chunk = ARD ? (p.chunk_q + AT - 1) / AT : (p.chunk_q + TT - 1) / TT;
  aa.W1 = sh + 2 * n;
  aa.w1_pair_stride = 4 * n;
  aa.w1_chunk_stride = 0;
  aa.rh = rh;
  aa.O = O;
  aa.npairs = P;
  aa.ntiles = aa.tiles_per_chunk;

  GradArgs ga{};
  ga.K = K;
  ga.V = V;
  ga.eta = eta;
  ga.tok_pair_stride = (int64_t)p.Nk * H;
  ga.eta_pair_stride = p.Nk;
  const int ntile = (p.chunk_kv + TT - 1) / TT;
  const int tiles_per_seg = (ntile + S - 1) / S;
  ga.seg_len = tiles_per_seg * TT;
  if (WS && nch > 0) {  // the role-split gradient kernel reads its segments' step-size scales
    LaunchTimer lt(K_LACT_INIT, st);
    hipLaunchKernelGGL(lact_eta_scale_kernel, dim3((unsigned)P, (unsigned)nch), dim3(256), 0, st, eta,
                       (int64_t)p.Nk, p.chunk_kv, ga.seg_len, S, s.esc);
    TTT_HIP(hipGetLastError());
  }
  ga.W0T = sh;
  ga.W2T = sh + n;
  ga.W1 = sh + 2 * n;
  ga.w_pair_stride = 4 * n;
  ga.rh = rh;
  ga.out = s.part;
  ga.out_y_stride = (int64_t)P * 3 * n;
  ga.out_pair_stride = 3 * n;
  ga.out_mat_stride = n;

  UpdateArgs ua{};
  ua.s = s;
  ua.S = S;
  ua.mask = p.update_mask;
  ua.muon = p.muon;
  ua.weight_norm = p.weight_norm;
  ua.momentum = p.momentum;
  ua.eps_norm = p.eps_norm;
  ua.eps_ns = p.eps_ns;

  // update path: LDS-resident kernel for the (h, rh) shapes it is built for, else the tiled launches
  const void* uk = nullptr;
  int ulds = 0;
  const void* uak = nullptr;  // update + apply in one launch
#define TTT_UPD(HH, RR)                                                                         \
  if (H == HH && rh == RR) {                                                                    \
    uk = reinterpret_cast<const void*>(lact_update_kernel<OpT, HH, RR>);                        \
    ulds = update_lds_bytes<HH, RR>();                                                          \
    if constexpr (ARD) uak = reinterpret_cast<const void*>(lact_update_apply_kernel<IoT, OpT, HH, RR>); \
  }
  // With Muon the LDS kernel evaluates Newton-Schulz through the h x h Gram matrix, whose
  // rounding grows with the conditioning of the write (weak directions are amplified by up to
  // 3.4445^5). It is used for 16-bit I/O when a chunk has at least h tokens (the write can have
  // full rank); fp32 I/O and shorter chunks keep the five explicit X rounds (tiled launches).
  const bool gram_ok = !p.muon || (sizeof(OpT) == 2 && p.chunk_kv >= H);
  if (gram_ok) {
    if constexpr (H == 32) { TTT_UPD(32, 64) TTT_UPD(32, 128) }
    if constexpr (H == 64) { TTT_UPD(64, 128) TTT_UPD(64, 256) }
    if constexpr (H == 96) { TTT_UPD(96, 192) TTT_UPD(96, 384) }
    if constexpr (H == 128) { TTT_UPD(128, 256) }
  }
#undef TTT_UPD
  if (uk) {
    TTT_HIP(hipFuncSetAttribute(uk, hipFuncAttributeMaxDynamicSharedMemorySize, ulds));
  }
  const bool fuse_ua = uak && p.order == TTT_APPLY_THEN_UPDATE;
  const int ualds = std::max(ulds, alds);
  if (fuse_ua) {
    TTT_HIP(hipFuncSetAttribute(uak, hipFuncAttributeMaxDynamicSharedMemorySize, ualds));
  }
  const unsigned ugrid = (unsigned)(3 * P);
  const int nupd = 8 * ((3 * P + 7) / 8);  // keeps the apply's workgroup -> XCD mapping

  const dim3 agrid(8u * (unsigned)((P + 7) / 8) * (unsigned)aa.ntiles);
  auto apply = [&]() -> ttt_status {
    LaunchTimer lt(K_LACT_APPLY, st);
    if constexpr (ARD)
      hipLaunchKernelGGL(akr, agrid, dim3(512), alds, st, aa);
    else
      hipLaunchKernelGGL(ak, agrid, dim3(256), alds, st, aa);
    TTT_HIP(hipGetLastError());
    return TTT_OK;
  };
  auto set_apply_weights = [&](const OpT* b) {
    aa.W0T = b;
    aa.W2T = b + n;
    aa.W1 = b + 2 * n;
    aa.W1T = b + 3 * n;
  };
  for (int c = 0; c < nch; ++c) {
    const OpT* rd = sh + (c & 1) * shb;
    const OpT* wr = sh + ((c + 1) & 1) * shb;
    set_apply_weights(rd);
    ga.W0T = rd;
    ga.W2T = rd + n;
    ga.W1 = rd + 2 * n;
    ua.s.sh = const_cast<OpT*>(wr);
    aa.t_base = c * p.chunk_q;
    aa.t_limit = (c + 1) * p.chunk_q;
    if (p.order == TTT_APPLY_THEN_UPDATE && !fuse_ua) {
      const ttt_status e = apply();
      if (e != TTT_OK) return e;
    }
    ga.t_base = c * p.chunk_kv;
    ga.eta_scale = s.esc + (int64_t)c * P * S;
    ga.t_limit = (c + 1) * p.chunk_kv;
    {
      LaunchTimer lt(K_LACT_GRAD, st);
      if constexpr (WS) {
        const unsigned grid = (unsigned)(rh / RB) * 8u * (unsigned)((P * S + 7) / 8);
        hipLaunchKernelGGL(gkw, dim3(grid), dim3(512), glds, st, ga, S, P);
      } else if constexpr (RD) {
        const unsigned grid = (unsigned)(rh / RB) * 8u * (unsigned)((P * S + 7) / 8);
        hipLaunchKernelGGL(gkr, dim3(grid), dim3(256), glds, st, ga, S, P);
      } else {
        hipLaunchKernelGGL(gk, dim3(rh / RB, S, P), dim3(256), glds, st, ga);
      }
      TTT_HIP(hipGetLastError());
    }
    if (fuse_ua) {
      LaunchTimer lt(K_LACT_UPD_APPLY, st);
      int nu = nupd;
      void* args[] = {&ua, &aa, &nu};
      TTT_HIP(hipLaunchKernel(uak, dim3((unsigned)nupd + agrid.x), dim3(512), args, (size_t)ualds, st));
      continue;
    }
    {
      LaunchTimer lt(K_LACT_UPDATE, st);
      void* args[] = {&ua};
      if (uk) {
        TTT_HIP(hipLaunchKernel(uk, dim3(ugrid), dim3(512), args, (size_t)ulds, st));
      } else {
        TTT_HIP(tu_run<OpT>(ua, st));
      }
    }
    if (p.order == TTT_UPDATE_THEN_APPLY) {
      set_apply_weights(wr);
      const ttt_status e = apply();
      if (e != TTT_OK) return e;
    }
  }
  LaunchTimer lt_fin(K_LACT_FINAL, st);
  hipLaunchKernelGGL(lact_final_kernel, dim3((unsigned)(n / 1024), 3, P), dim3(256), 0, st, s, W0o, W1o, W2o,
                     Mo);
  TTT_HIP(hipGetLastError());
  return TTT_OK;
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_lact_forward(const ttt_lact_params* p, const void* Q, const void* K,
                                       const void* V, const float* eta, const float* W0,
                                       const float* W1, const float* W2, const float* M_in, void* O,
                                       float* W0_out, float* W1_out, float* W2_out, float* M_out,
                                       void* workspace, size_t* workspace_bytes, void* stream) {
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_lact_params& q = *p;
  if (q.B < 0 || q.H < 0 || q.Nq < 0 || q.Nk < 0 || q.h <= 0 || q.r <= 0 || q.chunk_q <= 0 ||
      q.chunk_kv <= 0)
    return TTT_ERR_ARG;
  if (q.order != TTT_APPLY_THEN_UPDATE && q.order != TTT_UPDATE_THEN_APPLY) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (q.update_mask & ~7u) return TTT_ERR_ARG;
  if (q.w_batch_stride < 0) return TTT_ERR_ARG;
  if (q.Nq % q.chunk_q || q.Nk % q.chunk_kv) return TTT_ERR_SHAPE;
  if (q.Nq / q.chunk_q != q.Nk / q.chunk_kv) return TTT_ERR_SHAPE;
  const int64_t rh64 = (int64_t)q.r * q.h;
  if (q.h % 32 || rh64 % 64 || rh64 > 1024) return TTT_ERR_SHAPE;
  if (q.w_batch_stride != 0 && q.w_batch_stride != (int64_t)q.H * rh64 * q.h) return TTT_ERR_SHAPE;
  const bool bf16 = q.dtype == TTT_BF16;
  if (bf16 ? (q.h > 192) : (q.h > 64)) return TTT_ERR_UNSUPPORTED;
  const int P = q.B * q.H, h = q.h, rh = (int)rh64;
  const int64_t n = rh64 * h;
  const int nch = q.chunk_kv ? q.Nk / q.chunk_kv : 0;
  const bool have_tokens = P > 0 && nch > 0;
  if (P > 0) {
    if (!W0 || !W1 || !W2) return TTT_ERR_ARG;
    if (have_tokens && (!Q || !K || !V || !eta || !O)) return TTT_ERR_ARG;
  }
  // segments of the token contraction. The gradient kernels hold one workgroup per CU, so the
  // grid runs in rounds of 256: take the fewest segments whose grid fills its rounds to >= 97 %
  // (else the best filling up to 64 segments); a grid that already covers the chip keeps one.
  const int ntile = (q.chunk_kv + TT - 1) / TT;
  const int per_seg = (rh / RB) * std::max(P, 1);
  int S = 1;
  if (per_seg < 256) {
    double best = 0.0;
    for (int s = 1; s <= std::min(ntile, 64); ++s) {
      const int64_t tot = (int64_t)per_seg * s, rounds = (tot + 255) / 256;
      const double fill = (double)tot / (double)(256 * rounds);
      if (fill > best + 1e-9) {
        best = fill;
        S = s;
      }
      if (fill >= 0.97) break;
    }
  }
  const size_t opsz = bf16 ? 2 : 4;
  WorkspacePlan plan;
  const size_t oW = plan.add((size_t)P * 3 * n * 4);
  const size_t oM = plan.add((size_t)P * 3 * n * 4);
  const int NU = std::max(rh, h);
  const size_t oNu = plan.add((size_t)P * 3 * NU * 4);
  const size_t oSh = plan.add((size_t)2 * P * 4 * n * opsz);
  const size_t oPart = plan.add((size_t)S * P * 3 * n * 4);
  const size_t oU = plan.add((size_t)P * 3 * n * 4);
  const int64_t NSZ = 4 * n + 2 * (int64_t)h * h + TU_SS;
  const size_t oNs = plan.add((size_t)P * 3 * NSZ * 4);
  const size_t oEsc = plan.add((size_t)nch * P * S * 4);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (P == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  LactState s;
  s.W = reinterpret_cast<float*>(ws + oW);
  s.M = reinterpret_cast<float*>(ws + oM);
  s.nu = reinterpret_cast<float*>(ws + oNu);
  s.sh = ws + oSh;
  s.part = reinterpret_cast<float*>(ws + oPart);
  s.U = reinterpret_cast<float*>(ws + oU);
  s.ns = reinterpret_cast<float*>(ws + oNs);
  s.esc = reinterpret_cast<float*>(ws + oEsc);
  s.P = P;
  s.h = h;
  s.rh = rh;
  s.NU = NU;
  s.NSZ = NSZ;
  ttt_lact_params qq = q;
  if (!have_tokens) {  // nothing to apply: the final state is the initial state
    qq.Nq = qq.Nk = 0;
  }
#define TTT_LACT_CASE(IOT, OPT, HH)                                                                  \
  case HH:                                                                                         \
    return lact_run<IOT, OPT, HH>(qq, s, S, Q, K, V, eta, W0, W1, W2, M_in, O, W0_out, W1_out, W2_out, \
                                  M_out, st);
  try {
    if (bf16) {
      switch (h) {
        TTT_LACT_CASE(bf16_t, _Float16, 32)
        TTT_LACT_CASE(bf16_t, _Float16, 64)
        TTT_LACT_CASE(bf16_t, _Float16, 96)
        TTT_LACT_CASE(bf16_t, _Float16, 128)
        TTT_LACT_CASE(bf16_t, _Float16, 160)
        TTT_LACT_CASE(bf16_t, _Float16, 192)
        default: return TTT_ERR_UNSUPPORTED;
      }
    } else {
      switch (h) {
        TTT_LACT_CASE(float, float, 32)
        TTT_LACT_CASE(float, float, 64)
        default: return TTT_ERR_UNSUPPORTED;
      }
    }
  } catch (...) {
    return TTT_ERR_HIP;
  }
#undef TTT_LACT_CASE
}
