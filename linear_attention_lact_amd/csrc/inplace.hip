// inplace.hip -- In-Place TTT down-projection update on gfx950 (ttt_inplace_down_forward).
//
// "In-Place Test-Time Training" reading notes, section 3.1 / Eq. 2 and section 3.2 / Eq. 4:
// per chunk i of C tokens,
//   Z_i = silu(H_i W_gate^T) * (H_i W_up^T)     GEMM with a SwiGLU epilogue (two B operands)
//   O_i = Z_i W_down^T                           GEMM, bf16 store
//   W_down += eta Vbar_i^T Z_i                   GEMM with an fp32 read-modify-write epilogue
// All three are "TN" products C[M x N] = A[M x K] B[N x K]^T with K-contiguous operands:
// Z is written both token-major (for the apply, contracting over d_hidden) and hidden-major
// (for the update, contracting over tokens); Vbar is transposed once per sequence.
#include "common.hpp"
#include "host.hpp"
#include "timing.hpp"

namespace ttt {

namespace gemm {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_LD = BK + 8;  // padded row (elements)
enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_RMW = 2 };

struct Args {
  const __bf16* A;  int64_t lda;    // [M][K]
  const __bf16* B0; int64_t ldb;    // [N][K]
  const __bf16* B1;                 // second B (SwiGLU up projection)
  int M, N, K;
  __bf16* C; int64_t ldc;           // STORE / SWIGLU row-major output [M][N]
  __bf16* Ct; int64_t ldct;         // SWIGLU transposed output [N][M]
  float* Wf; __bf16* Wsh; int64_t ldw;  // RMW state and shadow [M][N]
  float alpha;
};

template <int EPI>
constexpr int lds_bytes() {
  return (EPI == EPI_SWIGLU ? 3 : 2) * BM * LDS_LD * 2;
}

// grid: tiles of 128x128 (x over N tiles, y over M tiles). block 256 = 4 waves (2x2), each
// wave a 64x64 quadrant = 2x2 MFMA tiles of 32x32.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_tn_kernel(Args g) {
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* As = reinterpret_cast<__bf16*>(smem);  // [BM][LDS_LD]
  __bf16* Bs = As + BM * LDS_LD;                 // [NB][BN][LDS_LD]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // each thread moves 4 16-byte vectors per operand tile: rows r = tid/8 + 32*v, col 8*(tid%8)
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  u32x4 ra[4], rb[NB][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ra[v] = *reinterpret_cast<const u32x4*>(g.A + (int64_t)(m0 + lr + 32 * v) * g.lda + k0 + lc);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const __bf16* Bp = b == 0 ? g.B0 : g.B1;
        rb[b][v] = *reinterpret_cast<const u32x4*>(Bp + (int64_t)(n0 + lr + 32 * v) * g.ldb + k0 + lc);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      *reinterpret_cast<u32x4*>(As + (lr + 32 * v) * LDS_LD + lc) = ra[v];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<u32x4*>(Bs + (b * BN + lr + 32 * v) * LDS_LD + lc) = rb[b][v];
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
    sstore();
    __syncthreads();
    if (k0 + BK < g.K) gload(k0 + BK);  // overlaps the MFMAs below
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_LD + kk + (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[b][j] = *reinterpret_cast<const bf16x8*>(Bs + (b * BN + wn * 64 + j * 32 + (lane & 31)) * LDS_LD + kk +
                                                       (lane >> 5) * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    }
  }

  // epilogues: element (m, n) of tile (i, j): m = m0 + wm*64 + i*32 + acc_row, n = ... + acc_col
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int mb = m0 + wm * 64 + i * 32, nb = n0 + wn * 64 + j * 32;
      const int n = nb + acc_col(lane);
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __bf16 zv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            const float gt = acc[0][i][j][r], up = acc[1][i][j][r];
            zv[e] = static_cast<__bf16>(gt * sigmoidf_(gt) * up);
            g.C[(int64_t)(mb + acc_row(r, lane)) * g.ldc + n] = zv[e];
          }
          // 4 consecutive rows m -> 4 consecutive elements of row n of the transposed copy
          __bf16* dst = g.Ct + (int64_t)n * g.ldct + mb + acc_row(4 * q, lane);
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v4 = {zv[0], zv[1], zv[2], zv[3]};
          *reinterpret_cast<bf16x4*>(dst) = v4;
        }
      } else if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          g.C[(int64_t)(mb + acc_row(r, lane)) * g.ldc + n] = static_cast<__bf16>(acc[0][i][j][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t idx = (int64_t)(mb + acc_row(r, lane)) * g.ldw + n;
          const float v = g.Wf[idx] + g.alpha * acc[0][i][j][r];
          g.Wf[idx] = v;
          g.Wsh[idx] = static_cast<__bf16>(v);
        }
      }
    }
}
}  // namespace gemm

// fp32 -> bf16 shadow copy. grid-stride, 4 elements per thread step.
__global__ void __launch_bounds__(256) to_bf16_kernel(const float* src, __bf16* dst, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * blockDim.x * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[i + e] = static_cast<__bf16>(v[e]);
  }
}

// [R][C] bf16 -> [C][R] bf16 through a 64x64 LDS tile. grid (C/64, R/64), block 256.
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const __bf16* src, __bf16* dst, int R, int C) {
  __shared__ __bf16 tile[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    tile[r][c] = src[(int64_t)(r0 + r) * C + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i / 64, r = i % 64;
    dst[(int64_t)(c0 + c) * R + r0 + r] = tile[r][c];
  }
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_inplace_down_forward(const ttt_inplace_params* p, const void* Hs,
                                               const void* W_gate, const void* W_up,
                                               const float* W_down, const void* Vbar, void* O,
                                               float* W_down_out, void* workspace,
                                               size_t* workspace_bytes, void* stream) {
  using namespace gemm;
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_inplace_params& q = *p;
  if (q.B < 0 || q.N < 0 || q.d_model <= 0 || q.d_hidden <= 0 || q.chunk <= 0) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (q.wdown_batch_stride < 0) return TTT_ERR_ARG;
  if (q.dtype != TTT_BF16) return TTT_ERR_UNSUPPORTED;
  if (q.N % q.chunk) return TTT_ERR_SHAPE;
  if (q.d_model % 256 || q.d_hidden % 256 || q.chunk % 128) return TTT_ERR_SHAPE;
  const int64_t nW = (int64_t)q.d_model * q.d_hidden;
  if (q.wdown_batch_stride != 0 && q.wdown_batch_stride != nW) return TTT_ERR_SHAPE;
  if (q.B > 0 && !W_down) return TTT_ERR_ARG;
  if (q.B > 0 && q.N > 0 && (!Hs || !W_gate || !W_up || !Vbar || !O)) return TTT_ERR_ARG;
  WorkspacePlan plan;
  const size_t oWf = plan.add(W_down_out ? 0 : (size_t)nW * 4);
  const size_t oSh = plan.add((size_t)nW * 2);
  const size_t oVt = plan.add((size_t)q.d_model * q.N * 2);
  const size_t oZ = plan.add((size_t)q.chunk * q.d_hidden * 2);
  const size_t oZt = plan.add((size_t)q.chunk * q.d_hidden * 2);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  __bf16* Wsh = reinterpret_cast<__bf16*>(ws + oSh);
  __bf16* Vt = reinterpret_cast<__bf16*>(ws + oVt);
  __bf16* Z = reinterpret_cast<__bf16*>(ws + oZ);
  __bf16* Zt = reinterpret_cast<__bf16*>(ws + oZt);
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(gemm_tn_kernel<EPI_SWIGLU>, lds_bytes<EPI_SWIGLU>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_STORE>, lds_bytes<EPI_STORE>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_RMW>, lds_bytes<EPI_RMW>());
    return e;
  }();
  TTT_HIP(lds_ok);
  const __bf16* Hb = static_cast<const __bf16*>(Hs);
  const __bf16* Vb = static_cast<const __bf16*>(Vbar);
  __bf16* Ob = static_cast<__bf16*>(O);
  const int nch = q.N / q.chunk;
  for (int b = 0; b < q.B; ++b) {
    float* Wf = W_down_out ? W_down_out + (int64_t)b * nW : reinterpret_cast<float*>(ws + oWf);
    TTT_HIP(hipMemcpyAsync(Wf, W_down + (int64_t)b * q.wdown_batch_stride, (size_t)nW * 4,
                           hipMemcpyDeviceToDevice, st));
    if (nch == 0) continue;
    {
      LaunchTimer lt(K_INP_PREP, st);
      hipLaunchKernelGGL(to_bf16_kernel, dim3(2048), dim3(256), 0, st, Wf, Wsh, nW);
      TTT_HIP(hipGetLastError());
      hipLaunchKernelGGL(transpose_bf16_kernel, dim3(q.d_model / 64, q.N / 64), dim3(256), 0, st,
                         Vb + (int64_t)b * q.N * q.d_model, Vt, q.N, q.d_model);
      TTT_HIP(hipGetLastError());
    }
    for (int i = 0; i < nch; ++i) {
      const int64_t t0 = (int64_t)i * q.chunk;
      Args z{};
      z.A = Hb + ((int64_t)b * q.N + t0) * q.d_model;
      z.lda = q.d_model;
      z.B0 = static_cast<const __bf16*>(W_gate);
      z.B1 = static_cast<const __bf16*>(W_up);
      z.ldb = q.d_model;
      z.M = q.chunk;
      z.N = q.d_hidden;
      z.K = q.d_model;
      z.C = Z;
      z.ldc = q.d_hidden;
      z.Ct = Zt;
      z.ldct = q.chunk;
      {
        LaunchTimer lt(K_INP_Z, st);
        hipLaunchKernelGGL(gemm_tn_kernel<EPI_SWIGLU>, dim3(q.d_hidden / BN, q.chunk / BM), dim3(256),
                           lds_bytes<EPI_SWIGLU>(), st, z);
        TTT_HIP(hipGetLastError());
      }
      Args a{};
      a.A = Z;
      a.lda = q.d_hidden;
      a.B0 = Wsh;
      a.ldb = q.d_hidden;
      a.M = q.chunk;
      a.N = q.d_model;
      a.K = q.d_hidden;
      a.C = Ob + ((int64_t)b * q.N + t0) * q.d_model;
      a.ldc = q.d_model;
      {
        LaunchTimer lt(K_INP_APPLY, st);
        hipLaunchKernelGGL(gemm_tn_kernel<EPI_STORE>, dim3(q.d_model / BN, q.chunk / BM), dim3(256),
                           lds_bytes<EPI_STORE>(), st, a);
        TTT_HIP(hipGetLastError());
      }
      Args u{};
      u.A = Vt + t0;
      u.lda = q.N;
      u.B0 = Zt;
      u.ldb = q.chunk;
      u.M = q.d_model;
      u.N = q.d_hidden;
      u.K = q.chunk;
      u.Wf = Wf;
      u.Wsh = Wsh;
      u.ldw = q.d_hidden;
      u.alpha = q.eta;
      {
        LaunchTimer lt(K_INP_UPDATE, st);
        hipLaunchKernelGGL(gemm_tn_kernel<EPI_RMW>, dim3(q.d_hidden / BN, q.d_model / BM), dim3(256),
                           lds_bytes<EPI_RMW>(), st, u);
        TTT_HIP(hipGetLastError());
      }
    }
  }
  return TTT_OK;
}
