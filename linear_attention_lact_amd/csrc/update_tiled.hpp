// Weight update for the shapes the LDS-resident kernel (update.hpp) does not cover: h > 128,
// fp32 operands, or chunks shorter than h (where the Gram form of Newton-Schulz loses
// precision). Same quantities as lact_update_kernel -- gradient of the chunk loss summed over
// the token segments, momentum, Frobenius normalisation, five Newton-Schulz iterations (LaCT
// paper, Section 3 "Nonlinear fast weight updates", Muon with coefficients 3.4445, -4.7750,
// 2.0315), W -= update, L2 renormalisation over the input dimension, operand shadows -- but
// every step is its own launch whose 32 x 32 output tiles are spread over the whole chip
// instead of one workgroup per matrix.
//
// Newton-Schulz takes the explicit form X <- aX + (bA + cA^2) X with A = X X^T, X the h x rh
// transpose of the write. Operands are fp32 in an L2-resident scratch; with 16-bit I/O each
// product is the split-bf16 MFMA (hi*hi + hi*lo + lo*hi, fp32 accumulation), with fp32 I/O the
// fp32 MFMA (exact fp32 products: the iteration amplifies rounding in weak singular directions
// by up to 3.4445^5, which a 2^-16 split would carry into the result). A tile is 4 waves, each summing
// a quarter of the contraction; the quarters are added in wave order, so results do not depend
// on scheduling. A and B = bA + cA^2 are symmetric: their upper-triangle tiles are computed and
// mirrored.
#pragma once
#include "update.hpp"

namespace ttt {

constexpr int TU_SS = 2048;  // scratch floats for per-tile sums of squares (n / 1024 <= 2048)
constexpr int TU_HMAX = 1024;  // widest state row (h) the final kernels handle

struct NsView {
  float* X[2];  // [h][rh]
  float* Y[2];  // [rh][h] (state layout, Y = X^T)
  float* A;     // [h][h]
  float* B;     // [h][h]
  float* ss;    // [TU_SS]
};

__device__ __forceinline__ NsView ns_view(const LactState& s, int pair, int mat) {
  const int64_t n = (int64_t)s.rh * s.h, hh = (int64_t)s.h * s.h;
  float* p = s.ns + ((int64_t)pair * 3 + mat) * s.NSZ;
  NsView v;
  v.X[0] = p;
  v.X[1] = p + n;
  v.Y[0] = p + 2 * n;
  v.Y[1] = p + 3 * n;
  v.A = p + 4 * n;
  v.B = v.A + hh;
  v.ss = v.B + hh;
  return v;
}

// update mask bits: W0 = 1, W1 = 2, W2 = 4 (matrix index 0, 1, 2)
__device__ __forceinline__ bool tu_active(const UpdateArgs& u, int mat) { return (u.mask >> mat) & 1u; }

// gradient = -(sum of the token-segment partials, in segment order), momentum, and per-tile
// sums of squares for the normalisation. grid (n / 1024, 3, P), 256 threads x 4 elements.
__global__ void __launch_bounds__(256) tu_reduce_kernel(UpdateArgs u) {
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ float red[16];
  const int64_t n = (int64_t)s.rh * s.h;
  const int64_t base = ((int64_t)pair * 3 + mat) * n;
  const int64_t e = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  const int64_t seg_stride = (int64_t)s.P * 3 * n;
  f32x4 g = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < u.S; ++k) g += *reinterpret_cast<const f32x4*>(s.part + k * seg_stride + base + e);
  f32x4 v = -g;
  if (u.momentum != 0.f) {
    f32x4* m = reinterpret_cast<f32x4*>(s.M + base + e);
    v = u.momentum * *m + v;
    *m = v;
  }
  const NsView nv = ns_view(s, pair, mat);
  *reinterpret_cast<f32x4*>(nv.Y[0] + e) = v;
  if (u.muon) {
    const float ss = block_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3], red);
    if (threadIdx.x == 0) nv.ss[blockIdx.x] = ss;
  }
}

// X0 = U / (||U||_F + eps) in both layouts. grid (rh/32 * h/32, 3, P), one 32 x 32 tile each.
__global__ void __launch_bounds__(256) tu_scale_kernel(UpdateArgs u, int nss) {
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ float red[16];
  __shared__ float tile[32][33];
  const NsView nv = ns_view(s, pair, mat);
  float ss = 0.f;
  for (int i = threadIdx.x; i < nss; i += 256) ss += nv.ss[i];
  const float inv = 1.f / (sqrtf(block_sum(ss, red)) + u.eps_ns);
  const int hb = s.h / 32;
  const int jb = blockIdx.x / hb, cb = blockIdx.x % hb;
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  f32x4* yp = reinterpret_cast<f32x4*>(nv.Y[0] + (int64_t)(jb * 32 + r) * s.h + cb * 32 + c4);
  const f32x4 v = *yp * inv;
  *yp = v;
#pragma unroll
  for (int q = 0; q < 4; ++q) tile[r][c4 + q] = v[q];
  __syncthreads();
  const f32x4 t = {tile[c4][r], tile[c4 + 1][r], tile[c4 + 2][r], tile[c4 + 3][r]};
  *reinterpret_cast<f32x4*>(nv.X[0] + (int64_t)(cb * 32 + r) * s.rh + jb * 32 + c4) = t;
}

// One 32 x 32 output tile of a . b^T over K (both operands row-major with K along rows): wave w
// takes the 16-wide k-steps [w*nk/4, (w+1)*nk/4) and leaves its partial tile in part[w].
struct TuLds {
  float part[4][32][33];
  float tile[32][33];
};

template <bool EXACT>
__device__ __forceinline__ void tu_partial(TuLds& L, const float* a, int lda, const float* b, int ldb, int K) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nk = K / 16;
  const int k0 = (w * nk / 4) * 16, k1 = ((w + 1) * nk / 4) * 16;
  f32x16 acc;
  zero(acc);
  // operands of up to four K steps requested together (they come from L2), then split and used
  const float* ap = a + (lane & 31) * lda + (lane >> 5) * 8;
  const float* bp = b + (lane & 31) * ldb + (lane >> 5) * 8;
  for (int kb = k0; kb < k1; kb += 64) {
    f32x4 av[4][2], bv[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb + 16 * j;
      if (k < k1) {
        av[j][0] = *reinterpret_cast<const f32x4*>(ap + k);
        av[j][1] = *reinterpret_cast<const f32x4*>(ap + k + 4);
        bv[j][0] = *reinterpret_cast<const f32x4*>(bp + k);
        bv[j][1] = *reinterpret_cast<const f32x4*>(bp + k + 4);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (EXACT && kb + 16 * j < k1) {
        // fp32 MFMA, K step 2: in step e lane half g supplies element 8 g + e of its 8 loaded
        // values, the same permutation for both operands, so the 8 steps cover the 16 k
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j][e >> 2][e & 3], bv[j][e >> 2][e & 3], acc, 0, 0, 0);
      } else if (kb + 16 * j < k1) {
        bf16x8 ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = av[j][e >> 2][e & 3], y = bv[j][e >> 2][e & 3];
          const __bf16 xh = static_cast<__bf16>(x), yh = static_cast<__bf16>(y);
          ah[e] = xh;
          al[e] = static_cast<__bf16>(x - static_cast<float>(xh));
          bh[e] = yh;
          bl[e] = static_cast<__bf16>(y - static_cast<float>(yh));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) L.part[w][acc_row(r, lane)][acc_col(lane)] = acc[r];
  __syncthreads();
}
// the full product at (row, col) of the tile, quarters added in wave order
__device__ __forceinline__ float tu_sum(const TuLds& L, int row, int col) {
  return ((L.part[0][row][col] + L.part[1][row][col]) + L.part[2][row][col]) + L.part[3][row][col];
}

// upper-triangle tile index -> (ib, kb) with ib <= kb
__device__ __forceinline__ void tu_tri(int t, int hb, int& ib, int& kb) {
  ib = 0;
  while (t >= hb - ib) {
    t -= hb - ib;
    ++ib;
  }
  kb = ib + t;
}

// A = X X^T. grid (hb(hb+1)/2, 3, P).
template <bool EXACT>
__global__ void __launch_bounds__(256) tu_gram_kernel(UpdateArgs u, int cur) {
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ TuLds L;
  const NsView nv = ns_view(s, pair, mat);
  const int h = s.h, rh = s.rh;
  int ib, kb;
  tu_tri(blockIdx.x, h / 32, ib, kb);
  const float* X = nv.X[cur];
  tu_partial<EXACT>(L, X + (int64_t)ib * 32 * rh, rh, X + (int64_t)kb * 32 * rh, rh, rh);
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  f32x4 v, m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = tu_sum(L, r, c4 + q);
    m[q] = tu_sum(L, c4 + q, r);
  }
  *reinterpret_cast<f32x4*>(nv.A + (ib * 32 + r) * h + kb * 32 + c4) = v;
  if (ib != kb) *reinterpret_cast<f32x4*>(nv.A + (kb * 32 + r) * h + ib * 32 + c4) = m;
}

// B = b A + c A A (A symmetric, so (AA)[i][k] = sum_m A[i][m] A[k][m]). grid (hb(hb+1)/2, 3, P).
template <bool EXACT>
__global__ void __launch_bounds__(256) tu_poly_kernel(UpdateArgs u) {
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ TuLds L;
  const NsView nv = ns_view(s, pair, mat);
  const int h = s.h;
  int ib, kb;
  tu_tri(blockIdx.x, h / 32, ib, kb);
  tu_partial<EXACT>(L, nv.A + ib * 32 * h, h, nv.A + kb * 32 * h, h, h);
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  const f32x4 a = *reinterpret_cast<const f32x4*>(nv.A + (ib * 32 + r) * h + kb * 32 + c4);
  const f32x4 at = *reinterpret_cast<const f32x4*>(nv.A + (kb * 32 + r) * h + ib * 32 + c4);
  f32x4 v, m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = NS_B * a[q] + NS_C * tu_sum(L, r, c4 + q);
    m[q] = NS_B * at[q] + NS_C * tu_sum(L, c4 + q, r);
  }
  *reinterpret_cast<f32x4*>(nv.B + (ib * 32 + r) * h + kb * 32 + c4) = v;
  if (ib != kb) *reinterpret_cast<f32x4*>(nv.B + (kb * 32 + r) * h + ib * 32 + c4) = m;
}

// X' = a X + B X, written as X' [h][rh] and Y' = X'^T [rh][h]. grid (h/32 * rh/32, 3, P).
template <bool EXACT>
__global__ void __launch_bounds__(256) tu_xupd_kernel(UpdateArgs u, int cur) {
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ TuLds L;
  const NsView nv = ns_view(s, pair, mat);
  const int h = s.h, rh = s.rh, rb = rh / 32;
  const int ib = blockIdx.x / rb, jb = blockIdx.x % rb;
  tu_partial<EXACT>(L, nv.B + ib * 32 * h, h, nv.Y[cur] + (int64_t)jb * 32 * h, h, h);
  const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
  const int64_t xo = (int64_t)(ib * 32 + r) * rh + jb * 32 + c4;
  const f32x4 x = *reinterpret_cast<const f32x4*>(nv.X[cur] + xo);
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = NS_A * x[q] + tu_sum(L, r, c4 + q);
    L.tile[r][c4 + q] = v[q];
  }
  *reinterpret_cast<f32x4*>(nv.X[cur ^ 1] + xo) = v;
  __syncthreads();
  const f32x4 t = {L.tile[c4][r], L.tile[c4 + 1][r], L.tile[c4 + 2][r], L.tile[c4 + 3][r]};
  *reinterpret_cast<f32x4*>(nv.Y[cur ^ 1] + (int64_t)(jb * 32 + r) * h + ib * 32 + c4) = t;
}

// W -= update for 32 state rows; W0T / W2T rows are renormalised over their h inputs and their
// shadows written here. W1 is renormalised per column over all rh rows: this kernel leaves the
// block's column sums of squares in the scratch (A's space) and tu_final_w1_kernel finishes.
// grid (rh/32, 3, P), 256 threads: wave w takes rows 8w..8w+7, lane l columns 256 k + 4l..+3 of
// each 256-column part k of the row (one part up to h = 256).
template <class OpT>
__global__ void __launch_bounds__(256) tu_final_kernel(UpdateArgs u, int ucur) {
  constexpr int NPART = TU_HMAX / 256;
  const LactState& s = u.s;
  const int mat = blockIdx.y, pair = blockIdx.z;
  if (!tu_active(u, mat)) return;
  __shared__ float colp[4][TU_HMAX];
  const NsView nv = ns_view(s, pair, mat);
  const int h = s.h, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t n = (int64_t)s.rh * h;
  float* W = s.W + ((int64_t)pair * 3 + mat) * n;
  const float* U = nv.Y[ucur];
  const float* nu = s.nu + ((int64_t)pair * 3 + mat) * s.NU;
  OpT* dst = reinterpret_cast<OpT*>(s.sh) + (int64_t)pair * 4 * n + (mat == 0 ? 0 : 1) * n;
  const int nparts = (h + 255) / 256;
  f32x4 cs[NPART];
#pragma unroll
  for (int k = 0; k < NPART; ++k) cs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int rr = 0; rr < 8; ++rr) {
    const int j = blockIdx.x * 32 + w * 8 + rr;
    f32x4 v[NPART];
    float sq = 0.f;
#pragma unroll
    for (int k = 0; k < NPART; ++k) {
      const int c = 256 * k + lane * 4;
      v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < nparts && c < h)
        v[k] = *reinterpret_cast<const f32x4*>(W + (int64_t)j * h + c) -
               *reinterpret_cast<const f32x4*>(U + (int64_t)j * h + c);
      sq += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
    }
    if (mat != 1 && u.weight_norm) {
      const float f = nu[j] / (sqrtf(wave_sum(sq)) + u.eps_norm);
#pragma unroll
      for (int k = 0; k < NPART; ++k) v[k] = v[k] * f;
    }
#pragma unroll
    for (int k = 0; k < NPART; ++k) {
      const int c = 256 * k + lane * 4;
      if (mat == 1) cs[k] += v[k] * v[k];
      if (k < nparts && c < h) {
        *reinterpret_cast<f32x4*>(W + (int64_t)j * h + c) = v[k];
        if (mat != 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[(int64_t)j * h + c + q] = Mfma<OpT>::from_f32(v[k][q]);
        }
      }
    }
  }
  if (mat == 1 && u.weight_norm) {
#pragma unroll
    for (int k = 0; k < NPART; ++k) {
      const int c = 256 * k + lane * 4;
      if (k < nparts && c < h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) colp[w][c + q] = cs[k][q];
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < h; c += 256)
      nv.A[blockIdx.x * h + c] = ((colp[0][c] + colp[1][c]) + colp[2][c]) + colp[3][c];
  }
}

// W1: column renormalisation from the per-block sums, then the W1 and W1T shadows.
// grid (rh/32, P), 256 threads.
template <class OpT>
__global__ void __launch_bounds__(256) tu_final_w1_kernel(UpdateArgs u) {
  constexpr int CW = 192;  // columns per part of the transposed shadow write
  const LactState& s = u.s;
  const int pair = blockIdx.y;
  __shared__ float f[TU_HMAX];
  __shared__ float tile[32][CW + 1];
  const NsView nv = ns_view(s, pair, 1);
  const int h = s.h, rh = s.rh, rb = rh / 32;
  const int64_t n = (int64_t)rh * h;
  float* W = s.W + ((int64_t)pair * 3 + 1) * n;
  const float* nu = s.nu + ((int64_t)pair * 3 + 1) * s.NU;
  OpT* sh = reinterpret_cast<OpT*>(s.sh) + (int64_t)pair * 4 * n;
  for (int c = threadIdx.x; c < h; c += 256) {
    float fc = 1.f;
    if (u.weight_norm) {
      float acc = 0.f;
      for (int b = 0; b < rb; ++b) acc += nv.A[b * h + c];
      fc = nu[c] / (sqrtf(acc) + u.eps_norm);
    }
    f[c] = fc;
  }
  __syncthreads();
  const int j0 = blockIdx.x * 32;
  for (int c0 = 0; c0 < h; c0 += CW) {  // columns c0 .. c0 + cw - 1
    const int cw = min(CW, h - c0);
    for (int i = threadIdx.x; i < 32 * cw; i += 256) {
      const int r = i / cw, c = c0 + i % cw;
      const int64_t o = (int64_t)(j0 + r) * h + c;
      const float v = W[o] * f[c];
      W[o] = v;
      sh[2 * n + o] = Mfma<OpT>::from_f32(v);
      tile[r][c - c0] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 32 * cw; i += 256) {
      const int c = i / 32, r = i % 32;
      sh[3 * n + (int64_t)(c0 + c) * rh + j0 + r] = Mfma<OpT>::from_f32(tile[r][c]);
    }
    __syncthreads();  // the tile is rewritten by the next part
  }
}

// Launch sequence. The scratch holds, per matrix, X[2], Y[2] (rh*h each), A and B (h*h) and
// TU_SS floats.
template <class OpT>
static hipError_t tu_run(const UpdateArgs& ua, hipStream_t st) {
  const int P = ua.s.P, hb = ua.s.h / 32, rb = ua.s.rh / 32;
  if (P == 0 || !(ua.mask & 7u)) return hipSuccess;
  const unsigned nt = (unsigned)(hb * rb), ntri = (unsigned)(hb * (hb + 1) / 2);
  const dim3 blk(256);
  hipLaunchKernelGGL(tu_reduce_kernel, dim3(nt, 3, P), blk, 0, st, ua);
  int cur = 0;
  if (ua.muon) {
    hipLaunchKernelGGL(tu_scale_kernel, dim3(nt, 3, P), blk, 0, st, ua, (int)nt);
    for (int it = 0; it < NS_STEPS; ++it) {
      constexpr bool EXACT = std::is_same<OpT, float>::value;
      hipLaunchKernelGGL(tu_gram_kernel<EXACT>, dim3(ntri, 3, P), blk, 0, st, ua, cur);
      hipLaunchKernelGGL(tu_poly_kernel<EXACT>, dim3(ntri, 3, P), blk, 0, st, ua);
      hipLaunchKernelGGL(tu_xupd_kernel<EXACT>, dim3(nt, 3, P), blk, 0, st, ua, cur);
      cur ^= 1;
    }
  }
  hipLaunchKernelGGL(tu_final_kernel<OpT>, dim3((unsigned)rb, 3, P), blk, 0, st, ua, cur);
  if (ua.mask & 2u) hipLaunchKernelGGL(tu_final_w1_kernel<OpT>, dim3((unsigned)rb, P), blk, 0, st, ua);
  return hipGetLastError();
}

}  // namespace ttt
