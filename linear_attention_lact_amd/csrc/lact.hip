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
#include "lact_large.hpp"
#include "timing.hpp"
#include "update.hpp"
#include "update_tiled.hpp"

namespace ttt {

// ---------------------------------------------------------------------------------------
// init: the initial state (W0, W2 transposed into rows of hidden units), momentum and both
// operand shadow buffers (a matrix outside the update mask keeps its initial shadow in each).
// grid (rh/32 * h/32, 3, P), block 256: one 32 x 32 tile of the state (rows j, columns c);
// W0/W2 and their momentum arrive in row form [h][rh] and are transposed through LDS.
// With flags (reset mode, before chunk c): only the pairs whose sequence has TTT_CHUNK_RESET set
// at chunk c return to the initial weights, with zero momentum (M_in is then null).
template <class OpT>
__device__ __forceinline__ void lact_init_tile(const LactState& s, const float* W0, const float* W1, const float* W2,
                                               const float* M_in, int H, int64_t w_batch_stride,
                                               const uint8_t* flags, int nch, int c, int tile, int mat, int pair) {
  __shared__ float tw[32][33], tm[32][33];
  const int h = s.h, rh = s.rh, hb = h / 32;
  const int64_t n = (int64_t)rh * h;
  const int j0 = (tile / hb) * 32, c0 = (tile % hb) * 32;
  const int b = pair / H, head = pair % H;
  if (flags && !(flags[(int64_t)b * nch + c] & TTT_CHUNK_RESET)) return;
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
    store4(sh + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n + e, sv);
    if (mat == 1)  // W1^T [h][rh]: row c0 + r, columns j0 + c4..
      store4(sh + 3 * n + (int64_t)(c0 + r) * rh + j0 + c4,
             f32x4{tw[c4][r], tw[c4 + 1][r], tw[c4 + 2][r], tw[c4 + 3][r]});
  }
}

template <class OpT>
__global__ void __launch_bounds__(256) lact_init_kernel(LactState s, const float* W0, const float* W1,
                                                       const float* W2, const float* M_in, int H,
                                                       int64_t w_batch_stride, const uint8_t* flags, int nch,
                                                       int c) {
  lact_init_tile<OpT>(s, W0, W1, W2, M_in, H, w_batch_stride, flags, nch, c, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Apply-only chunks (TTT_CHUNK_NO_UPDATE at chunk c): before the chunk's writes the state and
// momentum of the flagged pairs are saved to bak [2][P][3][rh*h]; after them they are put back
// and the shadow buffer the next reads use (sh) is rebuilt from them, so the writes (computed for
// every pair of the launch) leave no trace on those pairs. grid (rh/32 * h/32, 3, P), block 256.
template <class OpT>
__global__ void __launch_bounds__(256) lact_hold_kernel(LactState s, float* bak, const uint8_t* flags, int nch, int c,
                                                       int H, int restore, OpT* sh) {
  __shared__ float tw[32][33];
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!(flags[(int64_t)(pair / H) * nch + c] & TTT_CHUNK_NO_UPDATE)) return;
  const int h = s.h, rh = s.rh, hb = h / 32;
  const int64_t n = (int64_t)rh * h;
  const int j0 = (blockIdx.x / hb) * 32, c0 = (blockIdx.x % hb) * 32;
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  const int64_t e = ((int64_t)pair * 3 + mat) * n + (int64_t)(j0 + r) * h + c0 + c4;
  float* bw = bak + e;
  float* bm = bak + (int64_t)s.P * 3 * n + e;
  if (!restore) {
    *reinterpret_cast<f32x4*>(bw) = *reinterpret_cast<const f32x4*>(s.W + e);
    *reinterpret_cast<f32x4*>(bm) = *reinterpret_cast<const f32x4*>(s.M + e);
    return;
  }
  const f32x4 v = *reinterpret_cast<const f32x4*>(bw);
  *reinterpret_cast<f32x4*>(s.W + e) = v;
  *reinterpret_cast<f32x4*>(s.M + e) = *reinterpret_cast<const f32x4*>(bm);
  OpT* d = sh + (int64_t)pair * 4 * n + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n + (int64_t)(j0 + r) * h + c0 + c4;
#pragma unroll
  for (int q = 0; q < 4; ++q) d[q] = Mfma<OpT>::from_f32(v[q]);
  if (mat == 1) {  // W1^T [h][rh]: row c0 + r, columns j0 + c4..
#pragma unroll
    for (int q = 0; q < 4; ++q) tw[r][c4 + q] = v[q];
    __syncthreads();
    OpT* dt = sh + (int64_t)pair * 4 * n + 3 * n + (int64_t)(c0 + r) * rh + j0 + c4;
#pragma unroll
    for (int q = 0; q < 4; ++q) dt[q] = Mfma<OpT>::from_f32(tw[c4 + q][r]);
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
// grid (3, P), block 256. With fewer than 256 columns the rows split into rs = 256 / cols
// stripes (when that divides them), one thread per (stripe, column), 16 loads in flight each;
// the stripes' partial sums add in stripe order through LDS.
__device__ __forceinline__ void lact_norms_body(const LactState& s, const float* W0, const float* W1, const float* W2,
                                                int H, int64_t w_batch_stride, int mat, int pair) {
  __shared__ float part[256];
  const int h = s.h, rh = s.rh;
  const int64_t n = (int64_t)rh * h;
  const int b = pair / H, head = pair % H;
  const float* src = (mat == 0 ? W0 : mat == 1 ? W1 : W2) + (int64_t)b * w_batch_stride + (int64_t)head * n;
  float* nu = s.nu + ((int64_t)pair * 3 + mat) * s.NU;
  const int cols = mat == 1 ? h : rh, rows = mat == 1 ? rh : h;  // row-form [rows][cols]
  int rs = cols < 256 ? 256 / cols : 1;
  while (rs > 1 && rows % rs) --rs;
  if (rs == 1) {
    for (int j = threadIdx.x; j < cols; j += 256) {
      float acc = 0.f;
#pragma unroll 16
      for (int r = 0; r < rows; ++r) acc += src[(int64_t)r * cols + j] * src[(int64_t)r * cols + j];
      nu[j] = sqrtf(acc);
    }
    return;
  }
  const int t = threadIdx.x, j = t % cols, g = t / cols, len = rows / rs;
  float acc = 0.f;
  if (g < rs) {
#pragma unroll 16
    for (int r = g * len; r < (g + 1) * len; ++r) acc += src[(int64_t)r * cols + j] * src[(int64_t)r * cols + j];
  }
  part[t] = acc;
  __syncthreads();
  if (t < cols) {
    float tot = 0.f;
    for (int q = 0; q < rs; ++q) tot += part[q * cols + t];
    nu[t] = sqrtf(tot);
  }
}

// power-of-two step-size scales of the gradient's token segments: for chunk c, pair p and
// segment g, 2^-floor(log2(max eta)) over the segment's tokens and the nrow step-size rows
// (one, or one per matrix; 1 when the maximum is 0). grid (P, nch), block 256; out [nch][P][S].
__device__ __forceinline__ void lact_eta_scale_body(const float* eta, int64_t eta_pair_stride, int64_t row_stride,
                                                    int nrow, int chunk, int seg_len, int S, float* out, int pair,
                                                    int c, int P) {
  __shared__ float red[16];
  const float* ep = eta + pair * eta_pair_stride;
  for (int g = 0; g < S; ++g) {
    const int t0 = c * chunk + g * seg_len, t1 = min(t0 + seg_len, (c + 1) * chunk);
    float mx = 0.f;
    for (int e = 0; e < nrow; ++e)
      for (int t = t0 + threadIdx.x; t < t1; t += 256) mx = fmaxf(mx, ep[e * row_stride + t]);
    mx = block_max(mx, red);
    if (threadIdx.x == 0) out[((int64_t)c * P + pair) * S + g] = mx > 0.f ? exp2f(-floorf(log2f(mx))) : 1.f;
  }
}

// The call's prologue in one launch: workgroups [0, G) build the initial state tiles
// (lact_init_tile, G = tiles * 3 * P), the next 3 P the renorm targets (lact_norms_body), and the
// last P * nch, when nch > 0, the gradient segments' step-size scales (lact_eta_scale_body).
struct PrologueArgs {
  const float* eta;
  int64_t eta_pair_stride, row_stride;
  int nrow, chunk, seg_len, S, nch;
  float* out;
};
template <class OpT>
__global__ void __launch_bounds__(256) lact_prologue_kernel(LactState s, const float* W0, const float* W1,
                                                           const float* W2, const float* M_in, int H,
                                                           int64_t w_batch_stride, int tiles, PrologueArgs e) {
  const int P = s.P, bid = blockIdx.x, g = tiles * 3 * P;
  if (bid < g) {
    lact_init_tile<OpT>(s, W0, W1, W2, M_in, H, w_batch_stride, nullptr, 0, 0, bid % tiles, (bid / tiles) % 3,
                        bid / (3 * tiles));
  } else if (bid < g + 3 * P) {
    lact_norms_body(s, W0, W1, W2, H, w_batch_stride, (bid - g) % 3, (bid - g) / 3);
  } else {
    const int b = bid - g - 3 * P;
    lact_eta_scale_body(e.eta, e.eta_pair_stride, e.row_stride, e.nrow, e.chunk, e.seg_len, e.S, e.out, b % P,
                        b / P, P);
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
static ttt_status lact_run(const ttt_lact_params& p, const LactState& s, int S, float* bak, const void* Q,
                           const void* K, const void* V, const float* eta, const float* W0,
                           const float* W1, const float* W2, const float* M_in, void* O, float* W0o,
                           float* W1o, float* W2o, float* Mo, hipStream_t st) {
  constexpr bool SCALE = sizeof(OpT) == 2;
  constexpr bool RD = H <= 128;  // register-direct gradient kernel
  constexpr bool WS = std::is_same<OpT, _Float16>::value && (H == 64 || H == 128);  // its role-split form
  // eta per matrix: the E3 instances of the gradient kernels
  typedef typename std::conditional<WS, IoT, bf16_t>::type WIoT;
  const bool e3 = p.eta_per_matrix != 0;
  // the LDS-staged gradient kernel at h = 192: eight waves, the contractions split over all of them
  constexpr int GW = H == 192 ? 8 : NWAVE;
  auto gk = e3 ? grad_kernel<IoT, OpT, H, false, SCALE, true, GW> : grad_kernel<IoT, OpT, H, false, SCALE, false, GW>;
  auto gkr = e3 ? grad_rd_kernel<IoT, OpT, (RD ? H : 128), false, SCALE, true>
                : grad_rd_kernel<IoT, OpT, (RD ? H : 128), false, SCALE, false>;
  auto gkw = e3 ? grad_ws_kernel<WIoT, _Float16, (WS ? H : 128), true, true>
                : grad_ws_kernel<WIoT, _Float16, (WS ? H : 128), true, false>;
  auto ak = apply_kernel<IoT, OpT, H>;
  // register-direct apply where its double-buffered weight blocks fit in LDS
  constexpr bool ARD = H <= 128 && apply_rd_lds_bytes<OpT, (H <= 128 ? H : 128)>() <= 160 * 1024;
  auto akr = apply_rd_kernel<IoT, OpT, (ARD ? H : 64)>;
  constexpr int glds1 = WS   ? grad_ws_lds_bytes<_Float16, (WS ? H : 128)>()
                        : RD ? grad_rd_lds_bytes<OpT, (RD ? H : 128), false>()
                             : grad_lds_bytes<OpT, H, false>();
  constexpr int glds3 = WS   ? grad_ws_lds_bytes<_Float16, (WS ? H : 128), true>()
                        : RD ? grad_rd_lds_bytes<OpT, (RD ? H : 128), false, true>()
                             : grad_lds_bytes<OpT, H, false, true>();
  constexpr int glds = glds3;  // the larger of the two
  constexpr int alds = ARD ? apply_rd_lds_bytes<OpT, (ARD ? H : 64)>() : apply_lds_bytes<OpT, H>();
  static_assert(glds <= 160 * 1024 && alds <= 160 * 1024, "LDS budget");
  static const hipError_t lds_ok = [&] {
    hipError_t e = hipSuccess;
    for (int v = 0; v < 2 && e == hipSuccess; ++v) {
      auto k = v ? grad_ws_kernel<WIoT, _Float16, (WS ? H : 128), true, true>
                 : grad_ws_kernel<WIoT, _Float16, (WS ? H : 128), true, false>;
      auto kr = v ? grad_rd_kernel<IoT, OpT, (RD ? H : 128), false, SCALE, true>
                  : grad_rd_kernel<IoT, OpT, (RD ? H : 128), false, SCALE, false>;
      auto kg = v ? grad_kernel<IoT, OpT, H, false, SCALE, true, GW> : grad_kernel<IoT, OpT, H, false, SCALE, false, GW>;
      e = WS ? allow_lds(k, glds) : RD ? allow_lds(kr, glds) : allow_lds(kg, glds);
    }
    return e != hipSuccess ? e : (ARD ? allow_lds(akr, alds) : allow_lds(ak, alds));
  }();
  TTT_HIP(lds_ok);
  const int gl = e3 ? glds3 : glds1;

  const int P = s.P, rh = s.rh;
  const int64_t n = (int64_t)rh * H;
  const int nch = p.Nk / p.chunk_kv;

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
  ga.eta_pair_stride = (int64_t)(e3 ? 3 : 1) * p.Nk;  // eta [pair][Nk] or [pair][3][Nk]
  ga.eta_mat_stride = p.Nk;
  const int ntile = (p.chunk_kv + TT - 1) / TT;
  const int tiles_per_seg = (ntile + S - 1) / S;
  ga.seg_len = tiles_per_seg * TT;
  {
    // initial state, renorm targets and (for the role-split gradient kernel, which reads them)
    // the segments' step-size scales, in one launch
    LaunchTimer lt(K_LACT_INIT, st);
    const int ne = WS ? nch : 0;
    const PrologueArgs pe{eta, ga.eta_pair_stride, (int64_t)p.Nk, e3 ? 3 : 1, p.chunk_kv, ga.seg_len, S, ne, s.esc};
    const int tiles = (int)(n / 1024);
    hipLaunchKernelGGL(lact_prologue_kernel<OpT>, dim3((unsigned)(tiles * 3 * P + 3 * P + P * ne)), dim3(256), 0,
                       st, s, W0, W1, W2, M_in, p.H, p.w_batch_stride, tiles, pe);
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
    if constexpr (ARD)
      TTT_HIP(launch_k(K_LACT_APPLY, akr, agrid, dim3(512), alds, st, aa));
    else
      TTT_HIP(launch_k(K_LACT_APPLY, ak, agrid, dim3(256), alds, st, aa));
    return TTT_OK;
  };
  auto set_apply_weights = [&](const OpT* b) {
    aa.W0T = b;
    aa.W2T = b + n;
    aa.W1 = b + 2 * n;
    aa.W1T = b + 3 * n;
  };
  // per-chunk flags (resets before the chunk, apply-only chunks held) and inner steps: the k-th
  // write of the call reads shadow buffer k & 1 and writes the other
  const uint8_t* flags = p.chunk_flags;
  const int steps = p.inner_steps > 1 ? p.inner_steps : 1;
  const dim3 tgrid((unsigned)(n / 1024), 3, P);
  int it = 0;
  for (int c = 0; c < nch; ++c) {
    if (flags) {
      LaunchTimer lt(K_LACT_INIT, st);
      hipLaunchKernelGGL(lact_init_kernel<OpT>, tgrid, dim3(256), 0, st, s, W0, W1, W2, nullptr, p.H,
                         p.w_batch_stride, flags, nch, c);
      TTT_HIP(hipGetLastError());
      hipLaunchKernelGGL(lact_hold_kernel<OpT>, tgrid, dim3(256), 0, st, s, bak, flags, nch, c, p.H, 0, nullptr);
      TTT_HIP(hipGetLastError());
    }
    set_apply_weights(sh + (it & 1) * shb);
    aa.t_base = c * p.chunk_q;
    aa.t_limit = (c + 1) * p.chunk_q;
    if (p.order == TTT_APPLY_THEN_UPDATE && !fuse_ua) {
      const ttt_status e = apply();
      if (e != TTT_OK) return e;
    }
    ga.t_base = c * p.chunk_kv;
    ga.eta_scale = s.esc + (int64_t)c * P * S;
    ga.t_limit = (c + 1) * p.chunk_kv;
    for (int k = 0; k < steps; ++k, ++it) {
      const OpT* rd = sh + (it & 1) * shb;
      const OpT* wr = sh + ((it + 1) & 1) * shb;
      ga.W0T = rd;
      ga.W2T = rd + n;
      ga.W1 = rd + 2 * n;
      ua.s.sh = const_cast<OpT*>(wr);
      {
        const unsigned grid = (unsigned)(rh / RB) * 8u * (unsigned)((P * S + 7) / 8);
        if constexpr (WS)
          TTT_HIP(launch_k(K_LACT_GRAD, gkw, dim3(grid), dim3(512), gl, st, ga, S, P));
        else if constexpr (RD)
          TTT_HIP(launch_k(K_LACT_GRAD, gkr, dim3(grid), dim3(256), gl, st, ga, S, P));
        else
          TTT_HIP(launch_k(K_LACT_GRAD, gk, dim3(rh / RB, S, P), dim3(64 * GW), gl, st, ga));
      }
      if (fuse_ua && k == 0) {  // the chunk's apply reads the chunk-start weights (buffer rd)
        int nu = nupd;
        void* args[] = {&ua, &aa, &nu};
        TTT_HIP(launch_raw(K_LACT_UPD_APPLY, uak, dim3((unsigned)nupd + agrid.x), dim3(512), args, (size_t)ualds, st));
      } else if (uk) {
        void* args[] = {&ua};
        TTT_HIP(launch_raw(K_LACT_UPDATE, uk, dim3(ugrid), dim3(512), args, (size_t)ulds, st));
      } else {
        LaunchTimer lt(K_LACT_UPDATE, st);
        TTT_HIP(tu_run<OpT>(ua, st));
      }
    }
    if (flags) {
      LaunchTimer lt(K_LACT_INIT, st);
      hipLaunchKernelGGL(lact_hold_kernel<OpT>, tgrid, dim3(256), 0, st, s, bak, flags, nch, c, p.H, 1,
                         const_cast<OpT*>(sh + (it & 1) * shb));
      TTT_HIP(hipGetLastError());
    }
    if (p.order == TTT_UPDATE_THEN_APPLY) {
      set_apply_weights(sh + (it & 1) * shb);
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

// ---------------------------------------------------------------------------------------
// Heads wider than 192 (16-bit I/O): every chunk step composed of fp16 TN products
// (lact_large.hpp), one pair at a time, with the tiled update. Scratch of one pair, reused.
struct LargeWs {
  _Float16 *Kh, *Vh, *Kt, *Vt;  // chunk tokens [bk][h] and transposed [h][bk]
  float *Af, *Bf, *Df;          // forward products [bk][rh]
  _Float16 *EH, *X0, *X2;       // gradient intermediates, transposed [rh][bk]
  _Float16 *Qh, *Hq;            // apply: queries [bq][h], hidden [bq][rh]
};

static ttt_status lact_run_large(const ttt_lact_params& p, const LactState& s, const LargeWs& L, const void* Q,
                                 const void* K, const void* V, const float* eta, const float* W0, const float* W1,
                                 const float* W2, const float* M_in, void* O, float* W0o, float* W1o, float* W2o,
                                 float* Mo, hipStream_t st) {
  using namespace large;
  typedef _Float16 f16;
  const int P = s.P, h = s.h, rh = s.rh, bq = p.chunk_q, bk = p.chunk_kv;
  const int64_t n = (int64_t)rh * h;
  const int nch = p.Nk / p.chunk_kv;
  {
    LaunchTimer lt(K_LACT_INIT, st);
    const PrologueArgs pe{eta, (int64_t)p.Nk, (int64_t)p.Nk, 1, bk, bk, 1, nch, s.esc};
    const int tiles = (int)(n / 1024);
    hipLaunchKernelGGL(lact_prologue_kernel<f16>, dim3((unsigned)(tiles * 3 * P + 3 * P + P * nch)), dim3(256), 0,
                       st, s, W0, W1, W2, M_in, p.H, p.w_batch_stride, tiles, pe);
    TTT_HIP(hipGetLastError());
  }
  auto gemm = [&](int epi, const f16* A, int64_t lda, const f16* B0, const f16* B1, int64_t ldb, int M, int N, int Kd,
                  void* C, int64_t ldc, const float* inv) -> hipError_t {
    GArgs g{};
    g.A = A;
    g.lda = lda;
    g.B0 = B0;
    g.B1 = B1;
    g.ldb = ldb;
    g.M = M;
    g.N = N;
    g.K = Kd;
    g.C = C;
    g.ldc = ldc;
    g.alpha = 1.f;
    g.inv_dev = inv;
    const dim3 grid((unsigned)(N / BN), (unsigned)(M / BM));
    if (epi == G_F32) hipLaunchKernelGGL((gemm16_kernel<G_F32, float>), grid, dim3(256), lds_bytes<G_F32>(), st, g);
    else if (epi == G_SWI) hipLaunchKernelGGL((gemm16_kernel<G_SWI, f16>), grid, dim3(256), lds_bytes<G_SWI>(), st, g);
    else hipLaunchKernelGGL((gemm16_kernel<G_OUT, bf16_t>), grid, dim3(256), lds_bytes<G_OUT>(), st, g);
    return hipGetLastError();
  };
  const f16* sh = reinterpret_cast<const f16*>(s.sh);
  const int64_t shb = (int64_t)P * 4 * n;
  // O of chunk c from the weights in shadow buffer `buf`
  auto apply = [&](int c, const f16* buf) -> hipError_t {
    LaunchTimer lt(K_LACT_APPLY, st);
    for (int pr = 0; pr < P; ++pr) {
      const int64_t t0 = (int64_t)pr * p.Nq + (int64_t)c * bq;
      const f16* w = buf + (int64_t)pr * 4 * n;  // W0T, W2T, W1, W1T
      hipLaunchKernelGGL(tok16_kernel, dim3((unsigned)(h / 32), (unsigned)(bq / 32)), dim3(256), 0, st,
                         static_cast<const bf16_t*>(Q) + t0 * h, h, L.Qh, static_cast<f16*>(nullptr), (int64_t)0);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = gemm(G_SWI, L.Qh, h, w, w + n, h, bq, rh, h, L.Hq, rh, nullptr);
      if (e == hipSuccess) e = gemm(G_OUT, L.Hq, rh, w + 3 * n, nullptr, rh, bq, h, rh, static_cast<bf16_t*>(O) + t0 * h, h,
                                    nullptr);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  // segment partials (one segment) of chunk c at the weights in shadow buffer `buf`
  auto grad = [&](int c, const f16* buf) -> hipError_t {
    LaunchTimer lt(K_LACT_GRAD, st);
    for (int pr = 0; pr < P; ++pr) {
      const int64_t t0 = (int64_t)pr * p.Nk + (int64_t)c * bk;
      const f16* w = buf + (int64_t)pr * 4 * n;
      const dim3 tg((unsigned)(h / 32), (unsigned)(bk / 32));
      hipLaunchKernelGGL(tok16_kernel, tg, dim3(256), 0, st, static_cast<const bf16_t*>(K) + t0 * h, h, L.Kh, L.Kt,
                         (int64_t)bk);
      hipLaunchKernelGGL(tok16_kernel, tg, dim3(256), 0, st, static_cast<const bf16_t*>(V) + t0 * h, h, L.Vh, L.Vt,
                         (int64_t)bk);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = gemm(G_F32, L.Kh, h, w, nullptr, h, bk, rh, h, L.Af, rh, nullptr);          // K W0
      if (e == hipSuccess) e = gemm(G_F32, L.Kh, h, w + n, nullptr, h, bk, rh, h, L.Bf, rh, nullptr);      // K W2
      if (e == hipSuccess) e = gemm(G_F32, L.Vh, h, w + 2 * n, nullptr, h, bk, rh, h, L.Df, rh, nullptr);  // V W1^T
      if (e != hipSuccess) return e;
      const float* sc = s.esc + (int64_t)c * P + pr;
      hipLaunchKernelGGL(lgrad_epi_kernel, dim3((unsigned)(rh / 32), (unsigned)(bk / 32)), dim3(256), 0, st, L.Af,
                         L.Bf, L.Df, eta + t0, sc, rh, bk, L.EH, L.X0, L.X2);
      e = hipGetLastError();
      float* part = s.part + (int64_t)pr * 3 * n;  // P0, P1, P2 of this pair (rows j, columns c)
      if (e == hipSuccess) e = gemm(G_F32, L.EH, bk, L.Vt, nullptr, bk, rh, h, bk, part + n, h, sc);      // (eta H)^T V
      if (e == hipSuccess) e = gemm(G_F32, L.X0, bk, L.Kt, nullptr, bk, rh, h, bk, part, h, sc);          // X0^T K
      if (e == hipSuccess) e = gemm(G_F32, L.X2, bk, L.Kt, nullptr, bk, rh, h, bk, part + 2 * n, h, sc);  // X2^T K
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  UpdateArgs ua{};
  ua.s = s;
  ua.S = 1;
  ua.mask = p.update_mask;
  ua.muon = p.muon;
  ua.weight_norm = p.weight_norm;
  ua.momentum = p.momentum;
  ua.eps_norm = p.eps_norm;
  ua.eps_ns = p.eps_ns;
  for (int c = 0; c < nch; ++c) {
    const f16* rd = sh + (c & 1) * shb;
    const f16* wr = sh + ((c + 1) & 1) * shb;
    if (p.order == TTT_APPLY_THEN_UPDATE) TTT_HIP(apply(c, rd));
    TTT_HIP(grad(c, rd));
    ua.s.sh = const_cast<f16*>(wr);
    {
      LaunchTimer lt(K_LACT_UPDATE, st);
      TTT_HIP(tu_run<f16>(ua, st));
    }
    if (p.order == TTT_UPDATE_THEN_APPLY) TTT_HIP(apply(c, wr));
  }
  LaunchTimer lt_fin(K_LACT_FINAL, st);
  hipLaunchKernelGGL(lact_final_kernel, dim3((unsigned)(n / 1024), 3, P), dim3(256), 0, st, s, W0o, W1o, W2o, Mo);
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
  // heavy-ball coefficient in [0, 1), epsilons finite and >= 0 (the comparisons reject NaN)
  if (!(q.momentum >= 0.f && q.momentum < 1.f)) return TTT_ERR_ARG;
  if (!(q.eps_norm >= 0.f && q.eps_norm <= FLT_MAX) || !(q.eps_ns >= 0.f && q.eps_ns <= FLT_MAX)) return TTT_ERR_ARG;
  if (q.inner_steps < 0 || q.inner_steps > 64) return TTT_ERR_ARG;
  if (q.eta_per_matrix != 0 && q.eta_per_matrix != 1) return TTT_ERR_ARG;
  if (q.Nq % q.chunk_q || q.Nk % q.chunk_kv) return TTT_ERR_SHAPE;
  if (q.Nq / q.chunk_q != q.Nk / q.chunk_kv) return TTT_ERR_SHAPE;
  const int64_t rh64 = (int64_t)q.r * q.h;
  const bool bf16 = q.dtype == TTT_BF16;
  // heads wider than the LDS-resident kernels hold: the composed path (16-bit I/O)
  const bool large = bf16 && q.h > 192;
  if (q.h % 32 || rh64 % 64 || rh64 > (large ? 2048 : 1024)) return TTT_ERR_SHAPE;
  if (q.w_batch_stride != 0 && q.w_batch_stride != (int64_t)q.H * rh64 * q.h) return TTT_ERR_SHAPE;
  if (!bf16 && q.h > 64) return TTT_ERR_UNSUPPORTED;
  if (large) {
    if (q.h > TU_HMAX || q.chunk_flags || q.inner_steps > 1 || q.eta_per_matrix) return TTT_ERR_UNSUPPORTED;
    if (q.h % 128 || rh64 % 128 || q.chunk_q % 128 || q.chunk_kv % 128 || rh64 * q.h / 1024 > TU_SS)
      return TTT_ERR_SHAPE;
  }
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
  const size_t oBak = q.chunk_flags ? plan.add((size_t)2 * P * 3 * n * 4) : 0;  // held state of apply-only chunks
  size_t oL[12] = {0};
  if (large) {  // one pair's scratch of the composed path
    const size_t bk = (size_t)q.chunk_kv, bq = (size_t)q.chunk_q, hh = (size_t)h, rr = (size_t)rh;
    for (int i = 0; i < 4; ++i) oL[i] = plan.add(bk * hh * 2);       // Kh, Vh, Kt, Vt
    for (int i = 4; i < 7; ++i) oL[i] = plan.add(bk * rr * 4);       // Af, Bf, Df
    for (int i = 7; i < 10; ++i) oL[i] = plan.add(rr * bk * 2);      // EH, X0, X2
    oL[10] = plan.add(bq * hh * 2);                                   // Qh
    oL[11] = plan.add(bq * rr * 2);                                   // Hq
  }
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
    return lact_run<IOT, OPT, HH>(qq, s, S, q.chunk_flags ? reinterpret_cast<float*>(ws + oBak) : nullptr, Q, K, \
                                  V, eta, W0, W1, W2, M_in, O, W0_out, W1_out, W2_out, M_out, st);
  try {
    if (large) {
      auto f16p = [&](int i) { return reinterpret_cast<_Float16*>(ws + oL[i]); };
      auto f32p = [&](int i) { return reinterpret_cast<float*>(ws + oL[i]); };
      const LargeWs L{f16p(0), f16p(1), f16p(2), f16p(3), f32p(4), f32p(5), f32p(6),
                      f16p(7), f16p(8), f16p(9), f16p(10), f16p(11)};
      return lact_run_large(qq, s, L, Q, K, V, eta, W0, W1, W2, M_in, O, W0_out, W1_out, W2_out, M_out, st);
    }
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
