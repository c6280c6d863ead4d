// linattn_bwd.hip -- backward of the last-layer-only linear-attention form (ttt_linattn_backward).
//
// The forward is O_c = phi(Q_c) S_c with S_c = W1 + sum_j w(c, j) dS_j, dS_j = phi(K_j)^T
// diag(eta_j) V_j and phi(X) = silu(X W0) * (X W2) (KV-binding summary page, "Prerequisites ->
// Linear attention" and Theorems 5.2-5.3; press article, section 4: the parallel form the model
// trains through). With w the heavy-ball coefficients of the forward, given dO:
//   G_c = phi(Q_c)^T dO_c                      (the chunk-aggregate kernel with K := Q, V := dO)
//   R_j = sum_c w(c, j) G_c                    (a reverse heavy-ball scan per state element)
//   dW1 = sum_c G_c
//   query side, chunk c:  dphi = dO_c S_c^T
//   key side,   chunk j:  dphi = (eta V)_j R_j^T,  d(eta V)_j = phi(K_j) R_j,
//                         dV = eta d(eta V),  deta_t = <d(eta V)_t, V_t>
//   both: dA = dphi * Bm * silu'(A), dBm = dphi * silu(A) with A = X W0, Bm = X W2;
//         dX = dA W0^T + dBm W2^T,  dW0 += X^T dA,  dW2 += X^T dBm.
// The token kernel does the last three lines (and the key side's value gradients) for one
// (pair, chunk) per workgroup over 64-token tiles; its weight-gradient partials are added over
// chunks, the two sides and (for weights shared by the batch) the sequences by a fixed-order
// reduction.
#include "fastweight.hpp"
#include "host.hpp"
#include "linattn_scan.hpp"
#include "timing.hpp"

namespace ttt {

struct BwdTokArgs {
  const bf16_t* X;        // [pair][N][H] Q or K
  const bf16_t* L;        // [pair][N][H] dO (query side) or V (key side)
  const float* eta;       // [pair][N] (key side)
  const _Float16* M;      // [pair][nch][RH][H] S_c (query side) or R_c (key side), rows j
  const _Float16* W0T;    // [pair][RH][H] (W0^T, W2^T shadows, rows j)
  const _Float16* W2T;
  const _Float16* W0r;    // [pair][H][RH] row-form shadows
  const _Float16* W2r;
  bf16_t* dX;             // [pair][N][H]
  bf16_t* dV;             // [pair][N][H] (key side)
  float* deta;            // [pair][N] (key side)
  float* part;            // [pair][nch][2][H][RH] weight-gradient partials of this side
  int N, chunk, nch, P;
  int64_t wstride;        // elements between pairs of the weight shadows (= RH * H)
};

template <int H, int RH>
constexpr int bwd_tok_lds_bytes() {
  return (3 * TT * (H + 8) + 3 * TT * (RH + 8)) * 2 + (H / 32) * TT * 4;
}

// grid P * nch, block 256 (4 waves). KEY selects the key side.
template <int H, int RH, bool KEY>
__global__ void __launch_bounds__(256) linattn_bwd_tok_kernel(BwdTokArgs a) {
  typedef Mfma<_Float16> M;
  typedef M::frag frag;
  constexpr int LDX = H + 8, LDJ = RH + 8;
  constexpr int KS = H / M::KSTEP, KJ = RH / M::KSTEP, KT = TT / M::KSTEP;
  constexpr int TJ = RH / 32, TC = H / 32;
  constexpr int NT1 = 2 * TJ;               // [t][j] tiles of one token tile
  constexpr int NT4 = 2 * TC;               // [t][c] tiles
  constexpr int NT5 = 2 * TC * TJ;          // [c][j] tiles of dW0 and dW2
  constexpr int PW5 = (NT5 + 3) / 4;        // per wave
  static_assert(H % 32 == 0 && RH % 32 == 0 && NT5 <= 4 * 4, "shape");
  static_assert(4 % TJ == 0 && 4 % TC == 0, "a wave's tiles share one j block and one c block");

  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* Xs = reinterpret_cast<_Float16*>(smem);   // [TT][LDX]
  _Float16* Ls = Xs + TT * LDX;                        // [TT][LDX]
  _Float16* Ps = Ls + TT * LDX;                        // [TT][LDJ] phi (key side)
  _Float16* dAs = Ps + TT * LDJ;                       // [TT][LDJ]
  _Float16* dBs = dAs + TT * LDJ;                      // [TT][LDJ]
  bf16_t* Vs = reinterpret_cast<bf16_t*>(dBs + TT * LDJ);  // [TT][LDX] V as given (key side)
  float* red = reinterpret_cast<float*>(Vs + TT * LDX);      // [TC][TT] deta partials

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int pair = blockIdx.x / a.nch, c = blockIdx.x % a.nch;
  if (pair >= a.P) return;
  const int64_t tok = (int64_t)pair * a.N * H;
  const int cb = c * a.chunk, ce = cb + a.chunk;
  const int64_t n = (int64_t)RH * H;
  const _Float16* Mc = a.M + ((int64_t)pair * a.nch + c) * n;
  const _Float16* w0t = a.W0T + pair * a.wstride;
  const _Float16* w2t = a.W2T + pair * a.wstride;
  const _Float16* w0r = a.W0r + pair * a.wstride;
  const _Float16* w2r = a.W2r + pair * a.wstride;

  // the operand fragments of the fast weights and of the chunk's state that this wave's tiles
  // use: constant over the chunk, so loaded once (a wave's [t][j] tiles share the j block
  // w % TJ, its [t][c] tiles the c block w % TC)
  const int wj = w % TJ, wc = w % TC;
  frag w0f[KS], w2f[KS], mf[KS], w0rf[KJ], w2rf[KJ], mtf[KEY ? KJ : 1];
  {
    const int64_t jr = (int64_t)(wj * 32 + (lane & 31)) * H + (lane >> 5) * M::KSUB;
    const int64_t cr = (int64_t)(wc * 32 + (lane & 31)) * RH + (lane >> 5) * M::KSUB;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      w0f[s] = M::load(w0t + jr + s * M::KSTEP);
      w2f[s] = M::load(w2t + jr + s * M::KSTEP);
      mf[s] = M::load(Mc + jr + s * M::KSTEP);
    }
#pragma unroll
    for (int s = 0; s < KJ; ++s) {
      w0rf[s] = M::load(w0r + cr + s * M::KSTEP);
      w2rf[s] = M::load(w2r + cr + s * M::KSTEP);
      if constexpr (KEY) {
        // R^T rows c, K = j: gathered from the rows j of R (once per workgroup)
        const int cc = wc * 32 + (lane & 31), j0 = s * M::KSTEP + (lane >> 5) * M::KSUB;
#pragma unroll
        for (int e = 0; e < 8; ++e) mtf[s][e] = Mc[(int64_t)(j0 + e) * H + cc];
      }
    }
  }

  f32x16 acc5[PW5];
#pragma unroll
  for (int i = 0; i < PW5; ++i) zero(acc5[i]);

  // staging of X and L (key side: eta * V) through registers: the next tile is requested
  // before the current one is worked on
  constexpr int NCH = TT * H / 8 / 256;  // 16-byte chunks per thread and tensor
  static_assert(TT * H % (8 * 256) == 0, "staging map");
  u32x4 xg[NCH], lg[NCH];
  float eg[NCH];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int i = tid + 256 * k, r = i / (H / 8), col = (i % (H / 8)) * 8, t = t0 + r;
      xg[k] = lg[k] = u32x4{0u, 0u, 0u, 0u};
      eg[k] = 0.f;
      if (t < ce) {
        xg[k] = *reinterpret_cast<const u32x4*>(a.X + tok + (int64_t)t * H + col);
        lg[k] = *reinterpret_cast<const u32x4*>(a.L + tok + (int64_t)t * H + col);
        if (KEY) eg[k] = a.eta[(int64_t)pair * a.N + t];
      }
    }
  };
  fetch(cb);
  for (int t0 = cb; t0 < ce; t0 += TT) {
    // ---- stage X and L for tokens t0 .. t0 + 63 of the chunk; request the next tile ----
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int i = tid + 256 * k, r = i / (H / 8), col = (i % (H / 8)) * 8;
      *reinterpret_cast<f16x8*>(Xs + r * LDX + col) = bf16x8_to_f16x8(xg[k]);
      *reinterpret_cast<f16x8*>(Ls + r * LDX + col) = KEY ? bf16x8_scaled_f16x8(lg[k], eg[k]) : bf16x8_to_f16x8(lg[k]);
      if (KEY) *reinterpret_cast<u32x4*>(Vs + r * LDX + col) = lg[k];
    }
    if (t0 + TT < ce) fetch(t0 + TT);
    __syncthreads();

    // ---- A = X W0, Bm = X W2, D = L M^T per [t][j] tile; dA, dBm (and phi) to LDS ----
#pragma unroll
    for (int i = 0; i < (NT1 + 3) / 4; ++i) {
      const int q = w + 4 * i;
      if (q >= NT1) break;
      const int tt = q / TJ, tj = wj;
      f32x16 fa, fb, fd;
      zero(fa);
      zero(fb);
      zero(fd);
      const _Float16* xr = Xs + (tt * 32 + (lane & 31)) * LDX + (lane >> 5) * M::KSUB;
      const _Float16* lr = Ls + (tt * 32 + (lane & 31)) * LDX + (lane >> 5) * M::KSUB;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const frag xf = M::load(xr + s * M::KSTEP);
        fa = M::mma(xf, w0f[s], fa);
        fb = M::mma(xf, w2f[s], fb);
        fd = M::mma(M::load(lr + s * M::KSTEP), mf[s], fd);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tt * 32 + acc_row(r, lane), j = tj * 32 + acc_col(lane);
        const float A = fa[r], Bm = fb[r], D = fd[r];
        const float sg = 1.f / (1.f + __expf(-A));
        const float sil = A * sg;
        if (KEY) Ps[t * LDJ + j] = M::from_f32(sil * Bm);
        dAs[t * LDJ + j] = M::from_f32(D * Bm * (sg * (1.f + A * (1.f - sg))));
        dBs[t * LDJ + j] = M::from_f32(D * sil);
      }
    }
    __syncthreads();

    // ---- dX = dA W0^T + dBm W2^T per [t][c] tile; key side: d(eta V) = phi R, dV, deta ----
#pragma unroll
    for (int i = 0; i < (NT4 + 3) / 4; ++i) {
      const int q = w + 4 * i;
      if (q >= NT4) break;
      const int tt = q / TC, tc = wc;
      f32x16 fx;
      zero(fx);
      const _Float16* ar = dAs + (tt * 32 + (lane & 31)) * LDJ + (lane >> 5) * M::KSUB;
      const _Float16* br = dBs + (tt * 32 + (lane & 31)) * LDJ + (lane >> 5) * M::KSUB;
#pragma unroll
      for (int s = 0; s < KJ; ++s) {
        fx = M::mma(M::load(ar + s * M::KSTEP), w0rf[s], fx);
        fx = M::mma(M::load(br + s * M::KSTEP), w2rf[s], fx);
      }
      const int col = tc * 32 + acc_col(lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + tt * 32 + acc_row(r, lane);
        if (t < ce) Io<bf16_t>::store(a.dX + tok + (int64_t)t * H + col, fx[r]);
      }
      if constexpr (KEY) {
        f32x16 fe;
        zero(fe);
        const _Float16* pr = Ps + (tt * 32 + (lane & 31)) * LDJ + (lane >> 5) * M::KSUB;
#pragma unroll
        for (int s = 0; s < KJ; ++s) fe = M::mma(M::load(pr + s * M::KSTEP), mtf[s], fe);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tl = tt * 32 + acc_row(r, lane), t = t0 + tl;
          float dv = 0.f;
          if (t < ce) {
            const float e = a.eta[(int64_t)pair * a.N + t];
            Io<bf16_t>::store(a.dV + tok + (int64_t)t * H + col, e * fe[r]);
            dv = fe[r] * bf16_to_f32(Vs[tl * LDX + col].bits);
          }
          // sum over the tile's 32 columns (the lanes of one half-wave), in a fixed order
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) dv += __shfl_xor(dv, off, 64);
          if ((lane & 31) == 0) red[tc * TT + tl] = dv;
        }
      }
    }

    // ---- dW0 += X^T dA, dW2 += X^T dBm over the tile's tokens (K-major reads of both) ----
#pragma unroll
    for (int i = 0; i < PW5; ++i) {
      const int q = w + 4 * i;
      if (q < NT5) {
        const int m = q / (TC * TJ), rem = q % (TC * TJ), tc = rem / TJ, tj = rem % TJ;
        const _Float16* src = m == 0 ? dAs : dBs;
#pragma unroll
        for (int s = 0; s < KT; ++s)
          acc5[i] = M::mma(load_frag_tr<_Float16>(Xs + tc * 32, LDX, s * M::KSTEP, lane),
                           load_frag_tr<_Float16>(src + tj * 32, LDJ, s * M::KSTEP, lane), acc5[i]);
      }
    }
    __syncthreads();  // the tiles and the deta partials are complete
    if constexpr (KEY) {
      if (tid < TT && t0 + tid < ce) {
        float s = 0.f;
        for (int k = 0; k < TC; ++k) s += red[k * TT + tid];
        a.deta[(int64_t)pair * a.N + t0 + tid] = s;
      }
      __syncthreads();
    }
  }

  // ---- weight-gradient partials of this (pair, chunk) ----
  float* pp = a.part + ((int64_t)pair * a.nch + c) * 2 * (int64_t)H * RH;
#pragma unroll
  for (int i = 0; i < PW5; ++i) {
    const int q = w + 4 * i;
    if (q < NT5) {
      const int m = q / (TC * TJ), rem = q % (TC * TJ), tc = rem / TJ, tj = rem % TJ;
      float* o = pp + (int64_t)m * H * RH;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[(int64_t)(tc * 32 + acc_row(r, lane)) * RH + tj * 32 + acc_col(lane)] = acc5[i][r];
    }
  }
}

// Row-form fp32 weights W0, W2 [h][rh] of each pair to fp16 shadows (same layout).
// grid (ceil(n / 256), 2, P), block 256.
__global__ void __launch_bounds__(256) linattn_bwd_wrow_kernel(const float* W0, const float* W2, _Float16* out, int H,
                                                              int64_t n, int64_t w_batch_stride) {
  const int mat = blockIdx.y, pair = blockIdx.z;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int b = pair / H, head = pair % H;
  const float* src = (mat == 0 ? W0 : W2) + (int64_t)b * w_batch_stride + (int64_t)head * n;
  out[((int64_t)pair * 2 + mat) * n + e] = static_cast<_Float16>(src[e]);
}

// Reverse heavy-ball scan of the state gradients, one thread per state element [j][c]:
// R_j = T_j + alpha R_{j+1} with T_j = sum_{c > j} G_c (apply-then-update) or sum_{c >= j}
// (update-then-apply); writes R_j as fp16 rows [j][c] and the pair's dW1 = sum_c G_c
// (float32). grid (ceil(n / 256), P), block 256; the chunk increments are loaded eight at a time.
__global__ void __launch_bounds__(256) linattn_bwd_rscan_kernel(const float* G, _Float16* R, float* dW1p, int h,
                                                               int rh, int nch, int inclusive, float alpha) {
  const int pair = blockIdx.y;
  const int64_t n = (int64_t)rh * h;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const float* g = G + (int64_t)pair * nch * n + e;
  float T = 0.f, Rv = 0.f, tot = 0.f;
  for (int k0 = nch - 1; k0 >= 0; k0 -= 8) {
    float gk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) gk[u] = k0 - u >= 0 ? g[(int64_t)(k0 - u) * n] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 - u;
      if (k < 0) break;
      if (inclusive) T += gk[u];
      Rv = T + alpha * Rv;
      R[((int64_t)pair * nch + k) * n + e] = static_cast<_Float16>(Rv);
      if (!inclusive) T += gk[u];
      tot += gk[u];
    }
  }
  dW1p[(int64_t)pair * n + e] = tot;
}

// Weight gradients in the weights' layout: dW0 / dW2 [B?][H][h][rh] = sum over the sequences
// sharing the weights (all of them when w_batch_stride is 0, else one), the two sides and the
// chunks, in that fixed order; dW1 [B?][H][rh][h] likewise from the per-pair sums. Four
// consecutive elements per thread, the partials of eight chunks requested together.
// grid (ceil(n / 1024), 3, Hw) with Hw = H (shared) or B * H, block 256.
__global__ void __launch_bounds__(256) linattn_bwd_wreduce_kernel(const float* partq, const float* partk,
                                                                 const float* dW1p, float* dW0, float* dW2,
                                                                 float* dW1, int B, int H, int nch, int64_t n,
                                                                 int shared) {
  const int mat = blockIdx.y, slot = blockIdx.z;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  float* out = mat == 0 ? dW0 : mat == 1 ? dW2 : dW1;
  if (!out) return;
  const int nb = shared ? B : 1;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int bi = 0; bi < nb; ++bi) {
    const int pair = shared ? bi * H + slot : slot;
    if (mat == 2) {
      s += *reinterpret_cast<const f32x4*>(dW1p + (int64_t)pair * n + e);
      continue;
    }
    for (int side = 0; side < 2; ++side) {
      const float* p = (side == 0 ? partq : partk) + (int64_t)pair * nch * 2 * n + (int64_t)mat * n + e;
      for (int k0 = 0; k0 < nch; k0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = k0 + u < nch ? *reinterpret_cast<const f32x4*>(p + (int64_t)(k0 + u) * 2 * n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
    }
  }
  *reinterpret_cast<f32x4*>(out + (int64_t)slot * n + e) = s;
}

__global__ void __launch_bounds__(256) fill_kernel(float* p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int H, int RH>
static ttt_status linattn_bwd_run(const ttt_linattn_params& p, char* ws, const size_t* off, const void* Q,
                                  const void* K, const void* V, const float* eta, const float* W0, const float* W2,
                                  const float* W1, const void* dO, void* dQ, void* dK, void* dV, float* deta,
                                  float* dW0, float* dW2, float* dW1, hipStream_t st) {
  typedef _Float16 OpT;
  auto gkr = grad_rd_kernel<bf16_t, OpT, H, true, false>;
  constexpr int glds = grad_rd_lds_bytes<OpT, H, true>();
  constexpr int tlds = bwd_tok_lds_bytes<H, RH>();
  static_assert(glds <= 160 * 1024 && tlds <= 160 * 1024, "LDS budget");
  auto tq = linattn_bwd_tok_kernel<H, RH, false>;
  auto tk = linattn_bwd_tok_kernel<H, RH, true>;
  static const hipError_t lds_ok = [&] {
    hipError_t e = allow_lds(gkr, glds);
    if (e == hipSuccess) e = allow_lds(tq, tlds);
    return e != hipSuccess ? e : allow_lds(tk, tlds);
  }();
  TTT_HIP(lds_ok);
  const int P = p.B * p.H, nch = p.N / p.chunk;
  const int64_t n = (int64_t)RH * H;
  OpT* sh = reinterpret_cast<OpT*>(ws + off[0]);     // [P][2][RH][H] W0^T, W2^T
  OpT* wr = reinterpret_cast<OpT*>(ws + off[1]);     // [P][2][H][RH] W0, W2
  float* dS = reinterpret_cast<float*>(ws + off[2]); // [P][nch][n] forward aggregates, then G_c
  OpT* St = reinterpret_cast<OpT*>(ws + off[3]);     // [P][nch][n] forward states (rows)
  OpT* Rr = reinterpret_cast<OpT*>(ws + off[4]);     // [P][nch][n] R_c rows
  float* partq = reinterpret_cast<float*>(ws + off[6]);
  float* partk = reinterpret_cast<float*>(ws + off[7]);
  float* dW1p = reinterpret_cast<float*>(ws + off[8]);
  float* ones = reinterpret_cast<float*>(ws + off[9]);
  {
    LaunchTimer lt(K_LIN_PREP, st);
    hipLaunchKernelGGL(linattn_prep_kernel<OpT>, dim3((unsigned)((RH / 32) * (H / 32)), 2, P), dim3(256), 0, st, W0, W2,
                       sh, p.H, H, RH, p.w_batch_stride);
    TTT_HIP(hipGetLastError());
    hipLaunchKernelGGL(linattn_bwd_wrow_kernel, dim3((unsigned)((n + 255) / 256), 2, P), dim3(256), 0, st, W0, W2, wr,
                       p.H, n, p.w_batch_stride);
    TTT_HIP(hipGetLastError());
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0, st, ones, 1.f, (int64_t)p.N);
    TTT_HIP(hipGetLastError());
  }
  // forward aggregates and the states each chunk read
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
  ga.rh = RH;
  ga.out = dS;
  ga.out_y_stride = n;
  ga.out_pair_stride = (int64_t)nch * n;
  ga.out_mat_stride = 0;
  const unsigned ggrid = (unsigned)(RH / RB) * 8u * (unsigned)((P * nch + 7) / 8);
  TTT_HIP(launch_k(K_LIN_DELTA, gkr, dim3(ggrid), dim3(256), glds, st, ga, nch, P));
  {
    LaunchTimer lt(K_LIN_SCAN, st);
    auto sk = linattn_scan_kernel<OpT, true>;
    hipLaunchKernelGGL(sk, dim3((unsigned)((n + 255) / 256), P), dim3(256), 0, st, W1, dS,
                       St, nullptr, p.H, H, RH, nch, p.order == TTT_UPDATE_THEN_APPLY ? 1 : 0, p.momentum,
                       p.w_batch_stride, static_cast<const uint8_t*>(nullptr));
    TTT_HIP(hipGetLastError());
  }
  // G_c = phi(Q_c)^T dO_c: the aggregate kernel with K := Q, V := dO and unit step sizes
  GradArgs gq = ga;
  gq.K = Q;
  gq.V = dO;
  gq.eta = ones;
  gq.eta_pair_stride = 0;
  TTT_HIP(launch_k(K_LIN_DELTA, gkr, dim3(ggrid), dim3(256), glds, st, gq, nch, P));
  {
    LaunchTimer lt(K_LIN_SCAN, st);
    hipLaunchKernelGGL(linattn_bwd_rscan_kernel, dim3((unsigned)((n + 255) / 256), P), dim3(256), 0, st, dS, Rr,
                       dW1p, H, RH, nch, p.order == TTT_UPDATE_THEN_APPLY ? 1 : 0, p.momentum);
    TTT_HIP(hipGetLastError());
  }
  BwdTokArgs ta{};
  ta.W0T = sh;
  ta.W2T = sh + n;
  ta.W0r = wr;
  ta.W2r = wr + n;
  ta.wstride = 2 * n;
  ta.N = p.N;
  ta.chunk = p.chunk;
  ta.nch = nch;
  ta.P = P;
  BwdTokArgs aq = ta, ak = ta;
  aq.X = static_cast<const bf16_t*>(Q);
  aq.L = static_cast<const bf16_t*>(dO);
  aq.M = St;
  aq.dX = static_cast<bf16_t*>(dQ);
  aq.part = partq;
  ak.X = static_cast<const bf16_t*>(K);
  ak.L = static_cast<const bf16_t*>(V);
  ak.eta = eta;
  ak.M = Rr;
  ak.dX = static_cast<bf16_t*>(dK);
  ak.dV = static_cast<bf16_t*>(dV);
  ak.deta = deta;
  ak.part = partk;
  const dim3 tgrid((unsigned)(P * nch));
  TTT_HIP(launch_k(K_LIN_APPLY, tq, tgrid, dim3(256), tlds, st, aq));
  TTT_HIP(launch_k(K_LIN_APPLY, tk, tgrid, dim3(256), tlds, st, ak));
  {
    LaunchTimer lt(K_LIN_SCAN, st);
    const int shared = p.w_batch_stride == 0 ? 1 : 0;
    hipLaunchKernelGGL(linattn_bwd_wreduce_kernel, dim3((unsigned)((n + 1023) / 1024), 3, shared ? p.H : P), dim3(256), 0,
                       st, partq, partk, dW1p, dW0, dW2, dW1, p.B, p.H, nch, n, shared);
    TTT_HIP(hipGetLastError());
  }
  return TTT_OK;
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_linattn_backward(const ttt_linattn_params* p, const void* Q, const void* K, const void* V,
                                           const float* eta, const float* W0, const float* W2, const float* W1,
                                           const void* dO, void* dQ, void* dK, void* dV, float* deta, float* dW0,
                                           float* dW2, float* dW1, void* workspace, size_t* workspace_bytes,
                                           void* stream) {
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_linattn_params& q = *p;
  if (q.B < 0 || q.H < 0 || q.N < 0 || q.h <= 0 || q.r <= 0 || q.chunk <= 0) return TTT_ERR_ARG;
  if (q.order != TTT_APPLY_THEN_UPDATE && q.order != TTT_UPDATE_THEN_APPLY) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (q.w_batch_stride < 0) return TTT_ERR_ARG;
  if (!(q.momentum >= 0.f && q.momentum < 1.f)) return TTT_ERR_ARG;
  if (q.feature_map != TTT_PHI_SWIGLU && q.feature_map != TTT_PHI_IDENTITY) return TTT_ERR_ARG;
  if (q.N % q.chunk) return TTT_ERR_SHAPE;
  const int64_t rh64 = (int64_t)q.r * q.h;
  if (q.h % 32 || rh64 % 64 || rh64 > 1024) return TTT_ERR_SHAPE;
  if (q.w_batch_stride != 0 && q.w_batch_stride != (int64_t)q.H * rh64 * q.h) return TTT_ERR_SHAPE;
  // built: bf16, the SwiGLU map, (h, rh) in {(32, 64), (32, 128), (64, 128)}
  const bool shape_ok = (q.h == 32 && (rh64 == 64 || rh64 == 128)) || (q.h == 64 && rh64 == 128);
  if (q.dtype != TTT_BF16 || q.feature_map != TTT_PHI_SWIGLU || !shape_ok || q.chunk_flags) return TTT_ERR_UNSUPPORTED;
  const int P = q.B * q.H, nch = q.N / q.chunk;
  if (P > 0 && (!W0 || !W1 || !W2)) return TTT_ERR_ARG;
  if (P > 0 && nch > 0 && (!Q || !K || !V || !eta || !dO || !dQ || !dK || !dV || !deta)) return TTT_ERR_ARG;
  const int64_t n = rh64 * q.h;
  WorkspacePlan plan;
  size_t off[10];
  off[0] = plan.add((size_t)P * 2 * n * 2);
  off[1] = plan.add((size_t)P * 2 * n * 2);
  off[2] = plan.add((size_t)P * nch * n * 4);
  off[3] = plan.add((size_t)P * nch * n * 2);
  off[4] = plan.add((size_t)P * nch * n * 2);
  off[5] = plan.add(0);  // (unused)
  off[6] = plan.add((size_t)P * nch * 2 * n * 4);
  off[7] = plan.add((size_t)P * nch * 2 * n * 4);
  off[8] = plan.add((size_t)P * n * 4);
  off[9] = plan.add((size_t)std::max(q.N, 1) * 4);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (P == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int nw = q.w_batch_stride == 0 ? q.H : P;  // weight slots
  if (nch == 0) {  // no tokens: every gradient is zero (a fill kernel: safe under graph capture)
    for (float* d : {dW0, dW2, dW1}) {
      if (!d) continue;
      hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((nw * n + 255) / 256)), dim3(256), 0, st, d, 0.f, (int64_t)nw * n);
      TTT_HIP(hipGetLastError());
    }
    return TTT_OK;
  }
  char* ws = static_cast<char*>(workspace);
  try {
    if (q.h == 32 && rh64 == 64)
      return linattn_bwd_run<32, 64>(q, ws, off, Q, K, V, eta, W0, W2, W1, dO, dQ, dK, dV, deta, dW0, dW2, dW1, st);
    if (q.h == 32 && rh64 == 128)
      return linattn_bwd_run<32, 128>(q, ws, off, Q, K, V, eta, W0, W2, W1, dO, dQ, dK, dV, deta, dW0, dW2, dW1, st);
    return linattn_bwd_run<64, 128>(q, ws, off, Q, K, V, eta, W0, W2, W1, dO, dQ, dK, dV, deta, dW0, dW2, dW1, st);
  } catch (...) {
    return TTT_ERR_HIP;
  }
}
