// linattn_scan.hpp -- kernels shared by the multi-launch scan form and its backward: the
// operand shadows of W0 / W2 and the chunk prefix scan of the states each chunk reads.
#pragma once
#include "fastweight.hpp"
#include "host.hpp"

namespace ttt {

// Operand shadows W0T, W2T [rh][h] per pair from the row-form W0, W2 [h][rh]: one 32 x 32
// tile per workgroup, read along rows of W and written along rows of W^T through LDS.
// grid (rh/32 * h/32, 2, P), block 256 (each thread 4 elements).
template <class OpT>
__global__ void __launch_bounds__(256) linattn_prep_kernel(const float* __restrict__ W0, const float* __restrict__ W2,
                                                          OpT* __restrict__ sh, int H, int h, int rh,
                                                          int64_t w_batch_stride) {
  __shared__ float tile[32][33];
  const int mat = blockIdx.y, pair = blockIdx.z;
  const int tj = blockIdx.x % (rh / 32), tc = blockIdx.x / (rh / 32);  // tile of j (rh) and c (h)
  const int b = pair / H, head = pair % H;
  const int64_t n = (int64_t)rh * h;
  const float* src = (mat == 0 ? W0 : W2) + (int64_t)b * w_batch_stride + (int64_t)head * n;
  OpT* dst = sh + ((int64_t)pair * 2 + mat) * n;
  const int x = threadIdx.x % 32, y = threadIdx.x / 32;
#pragma unroll
  for (int k = 0; k < 4; ++k) tile[y + 8 * k][x] = src[(int64_t)(tc * 32 + y + 8 * k) * rh + tj * 32 + x];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k)
    dst[(int64_t)(tj * 32 + y + 8 * k) * h + tc * 32 + x] = Mfma<OpT>::from_f32(tile[x][y + 8 * k]);
}

// Chunk prefix scan, one thread per state element [j][c]: writes S_c per chunk as an operand
// shadow, [rh][h] (ROWS) or transposed [h][rh], and optionally the final state. With a
// momentum coefficient alpha each chunk's write passes through the heavy-ball buffer
// m <- alpha m + dS_k, s <- s + m, which gives chunk k's write the cumulative coefficient
// sum_{i>=k} alpha^(i-k) of Theorem 5.3; alpha = 0 leaves m = dS_k, the plain prefix.
// flags (nullable, [B][nch]): TTT_CHUNK_RESET restarts from W1 with m = 0 before chunk k,
// TTT_CHUNK_NO_UPDATE skips chunk k's write and its momentum step.
// grid (ceil(rh*h/256), P), block 256.
template <class OpT, bool ROWS>
__global__ void __launch_bounds__(256) linattn_scan_kernel(const float* __restrict__ W1, const float* __restrict__ dS,
                                                          OpT* __restrict__ St, float* __restrict__ S_out,
                                                          int H, int h, int rh, int nch, int inclusive,
                                                          float alpha, int64_t w_batch_stride,
                                                          const uint8_t* flags) {
  const int pair = blockIdx.y;
  const int64_t n = (int64_t)rh * h;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int b = pair / H, head = pair % H;
  const int j = (int)(e / h), c = (int)(e % h);
  const float s0 = W1[(int64_t)b * w_batch_stride + (int64_t)head * n + e];
  float s = s0, m = 0.f;
  const uint8_t* fl = flags ? flags + (int64_t)b * nch : nullptr;
  const float* d = dS + (int64_t)pair * nch * n + e;
  OpT* o = St + (int64_t)pair * nch * n + (ROWS ? e : (int64_t)c * rh + j);
  // the chunk increments are loaded eight at a time so that their latencies overlap
  for (int k0 = 0; k0 < nch; k0 += 8) {
    float dk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) dk[u] = k0 + u < nch ? d[(int64_t)(k0 + u) * n] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u >= nch) break;
      const int f = fl ? fl[k0 + u] : 0;
      if (f & TTT_CHUNK_RESET) {
        s = s0;
        m = 0.f;
      }
      const bool write = !(f & TTT_CHUNK_NO_UPDATE);
      if (inclusive && write) {
        m = fmaf(alpha, m, dk[u]);
        s += m;
      }
      o[(int64_t)(k0 + u) * n] = Mfma<OpT>::from_f32(s);
      if (!inclusive && write) {
        m = fmaf(alpha, m, dk[u]);
        s += m;
      }
    }
  }
  if (S_out) S_out[(int64_t)pair * n + e] = s;
}

}  // namespace ttt
