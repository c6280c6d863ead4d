// lact_large.hpp -- the LaCT chunk step for heads wider than the LDS-resident kernels hold
// (h > 192, 16-bit I/O), composed of plain TN products on fp16 MFMA operands.
//
// Per (sequence, head) pair and chunk ("Test-Time Training Done Right" reading notes, sections
// 2.1-2.2; the same quantities as the fast path):
//   forward of the write:  A = K W0, Bm = K W2, D = V W1^T          (three products, fp32 out)
//   gradient intermediates: eta*H = eta silu(A) Bm, X0 = eta D Bm silu'(A), X2 = eta D silu(A)
//                           (one elementwise kernel, written transposed, fp16)
//   token contractions:     P1 = (eta H)^T V, P0 = X0^T K, P2 = X2^T K  (K = chunk tokens)
//   apply:                  O = (silu(Q W0) * (Q W2)) W1            (two products)
// The update (momentum, Newton-Schulz, renorm, shadows) is the tiled one. As in the fast path,
// the step sizes are scaled by a power of two per (chunk, pair) before they enter fp16
// intermediates, and the contractions are scaled back.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace ttt {
namespace large {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_LD = BK + 8;  // padded row (fp16 elements)
enum { G_F32 = 0, G_OUT = 1, G_SWI = 2 };

struct GArgs {
  const _Float16* A; int64_t lda;   // [M][K]
  const _Float16* B0; int64_t ldb;  // [N][K]
  const _Float16* B1;               // second B (G_SWI: the up projection)
  int M, N, K;
  void* C; int64_t ldc;             // [M][N]: float (G_F32), OutT (G_OUT), fp16 (G_SWI)
  float alpha;                      // G_F32: C = alpha * acc ...
  const float* inv_dev;             // ... / *inv_dev when set (a device-side scale)
};

template <int EPI>
constexpr int lds_bytes() { return (EPI == G_SWI ? 3 : 2) * BM * LDS_LD * 2; }

// C = A B^T. grid (N / 128, M / 128), block 256 = 4 waves (2 x 2), each a 64 x 64 quadrant of
// 2 x 2 MFMA 32x32x16 f16 tiles. Operand tiles go global -> registers -> LDS, the next K block's
// loads in flight during the current block's products.
template <int EPI, class OutT>
__global__ void __launch_bounds__(256) gemm16_kernel(GArgs g) {
  constexpr int NB = EPI == G_SWI ? 2 : 1;
  typedef _Float16 f16;
  extern __shared__ __align__(16) unsigned char smem[];
  f16* As = reinterpret_cast<f16*>(smem);  // [BM][LDS_LD]
  f16* Bs = As + BM * LDS_LD;              // [NB][BN][LDS_LD]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // rows lr + 32 v, 8 columns from lc
  u32x4 ra[4], rb[NB][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ra[v] = *reinterpret_cast<const u32x4*>(g.A + (int64_t)(m0 + lr + 32 * v) * g.lda + k0 + lc);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        rb[b][v] = *reinterpret_cast<const u32x4*>((b == 0 ? g.B0 : g.B1) + (int64_t)(n0 + lr + 32 * v) * g.ldb +
                                                   k0 + lc);
    }
  };
  f32x16 acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) zero(acc[b][i][j]);
  gload(0);
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      *reinterpret_cast<u32x4*>(As + (lr + 32 * v) * LDS_LD + lc) = ra[v];
#pragma unroll
      for (int b = 0; b < NB; ++b) *reinterpret_cast<u32x4*>(Bs + (b * BN + lr + 32 * v) * LDS_LD + lc) = rb[b][v];
    }
    __syncthreads();
    if (k0 + BK < g.K) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      f16x8 af[2], bfr[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const f16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_LD + kk + (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[b][j] = *reinterpret_cast<const f16x8*>(Bs + (b * BN + wn * 64 + j * 32 + (lane & 31)) * LDS_LD + kk +
                                                      (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    }
  }
  float alpha = g.alpha;
  if (EPI == G_F32 && g.inv_dev) alpha /= *g.inv_dev;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int mb = m0 + wm * 64 + i * 32, n = n0 + wn * 64 + j * 32 + acc_col(lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t o = (int64_t)(mb + acc_row(r, lane)) * g.ldc + n;
        if constexpr (EPI == G_F32) {
          static_cast<float*>(g.C)[o] = alpha * acc[0][i][j][r];
        } else if constexpr (EPI == G_OUT) {
          if constexpr (std::is_same<OutT, bf16_t>::value)
            static_cast<bf16_t*>(g.C)[o].bits = f32_to_bf16(acc[0][i][j][r]);
          else
            static_cast<OutT*>(g.C)[o] = static_cast<OutT>(acc[0][i][j][r]);
        } else {
          const float gt = acc[0][i][j][r], up = acc[1][i][j][r];
          static_cast<f16*>(g.C)[o] = static_cast<f16>(gt * sigmoidf_(gt) * up);
        }
      }
    }
}

// Token rows [rows][h] (bf16) to fp16: row-major into dst (ld h) and, when dstT is set,
// transposed into dstT [h][ld_t] at column offset 0. grid (h / 32, rows / 32), block 256.
__global__ void __launch_bounds__(256) tok16_kernel(const bf16_t* __restrict__ src, int h, _Float16* __restrict__ dst,
                                                   _Float16* __restrict__ dstT, int64_t ld_t) {
  __shared__ float t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int i = threadIdx.x; i < 32 * 32; i += 256) {
    const int r = i / 32, c = i % 32;
    const float v = bf16_to_f32(src[(int64_t)(r0 + r) * h + c0 + c].bits);
    dst[(int64_t)(r0 + r) * h + c0 + c] = static_cast<_Float16>(v);
    t[r][c] = v;
  }
  if (!dstT) return;
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * 32; i += 256) {
    const int c = i / 32, r = i % 32;
    dstT[(int64_t)(c0 + c) * ld_t + r0 + r] = static_cast<_Float16>(t[r][c]);
  }
}

// Gradient intermediates of one pair and chunk from A, Bm, D (fp32 [b][rh]) and the chunk's step
// sizes eta [b] times the power-of-two *scale: eta*H, X0, X2 written transposed (fp16 [rh][b]).
// grid (rh / 32, b / 32), block 256.
__global__ void __launch_bounds__(256) lgrad_epi_kernel(const float* __restrict__ Af, const float* __restrict__ Bf,
                                                       const float* __restrict__ Df, const float* __restrict__ eta,
                                                       const float* __restrict__ scale, int rh, int b,
                                                       _Float16* __restrict__ EH, _Float16* __restrict__ X0,
                                                       _Float16* __restrict__ X2) {
  __shared__ float t0[32][33], t1[32][33], t2[32][33];
  const int j0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const float sc = *scale;
  for (int i = threadIdx.x; i < 32 * 32; i += 256) {
    const int r = i / 32, c = i % 32;
    const int64_t o = (int64_t)(r0 + r) * rh + j0 + c;
    const float A = Af[o], Bm = Bf[o], D = Df[o], e = eta[r0 + r] * sc;
    const float sg = sigmoidf_(A), sil = A * sg;
    t0[r][c] = e * sil * Bm;
    t1[r][c] = e * D * Bm * (sg * (1.f + A * (1.f - sg)));
    t2[r][c] = e * D * sil;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * 32; i += 256) {
    const int c = i / 32, r = i % 32;
    const int64_t o = (int64_t)(j0 + c) * b + r0 + r;
    EH[o] = static_cast<_Float16>(t0[r][c]);
    X0[o] = static_cast<_Float16>(t1[r][c]);
    X2[o] = static_cast<_Float16>(t2[r][c]);
  }
}

}  // namespace large
}  // namespace ttt
