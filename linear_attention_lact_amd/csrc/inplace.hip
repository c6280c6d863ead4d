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
#include <mutex>

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

// ---------------------------------------------------------------------------------------------
// Large-tile TN GEMM for shapes divisible by its tile: 256 x 256 outputs per workgroup (SwiGLU:
// 256 tokens x 128 hidden units for each of the two B operands), K in blocks of 64, 8 waves
// (2 per SIMD, so one wave's LDS reads overlap the other's MFMAs), each a 128 x 64 block of
// 4 x 2 MFMA 32x32x16 tiles. Operand tiles go global -> LDS directly (16-byte lane-contiguous
// DMA loads, no register staging), double-buffered: the loads of block k + 2 are issued once
// every wave is done with block k. LDS rows are 128 bytes (64 bf16); the 16-byte K chunk c of
// row r sits at position c ^ (r % 8) ^ ((r / 8) % 2), so the rows an MFMA operand read touches
// together fall into distinct bank groups. An optional K split writes fp32 partials that a
// second kernel adds in split order.
namespace gemm2 {
using gemm::Args;
using gemm::EPI_SWIGLU;
using gemm::EPI_STORE;
using gemm::EPI_RMW;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROWB = BK * 2;                    // bytes per staged row
constexpr int STAGE = (BM + BN) * ROWB;         // 64 KB: A rows, then B rows
constexpr int LDS = 2 * STAGE;
constexpr int THREADS = 512;
constexpr int EPI_PARTIAL = 3;                  // fp32 partial of one K split

template <int EPI>
constexpr int tile_n() { return EPI == EPI_SWIGLU ? BN / 2 : BN; }

__device__ __forceinline__ int chunk_pos(int c, int row) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

// grid: ksplit * (M / BM) * (N / tile_n) workgroups of 512 threads; split fastest, then N tile.
// Wave w: rows (w & 1) * 128.. of the A tile; B rows (w >> 1) * 64.. (SwiGLU: gate rows
// (w >> 1) * 32.. and the same up rows, so each wave holds both factors of its outputs).
template <int EPI>
__global__ void __launch_bounds__(512) gemm_big_kernel(Args g, int ksplit, float* part) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int TN = tile_n<EPI>();
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int ntn = g.N / TN;
  int bid = blockIdx.x;
  const int ks = bid % ksplit;
  bid /= ksplit;
  const int m0 = (bid / ntn) * BM, n0 = (bid % ntn) * TN;
  const int kper = g.K / ksplit, kbeg = ks * kper, nkb = kper / BK;

  // staging: instruction j of wave w fills rows 32w + 8j .. +8 of each operand tile; lane l
  // takes row + l/8 and LDS chunk l%8
  const int lr = lane >> 3;
  const __bf16* asrc[4];
  const __bf16* bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * w + 8 * j + lr;
    const int ch = chunk_pos(lane & 7, row);
    asrc[j] = g.A + (int64_t)(m0 + row) * g.lda + kbeg + ch * 8;
    // B tile rows: SwiGLU rows 0..127 gate, 128..255 up (same hidden units n0..n0+127)
    bsrc[j] = SW ? (row < 128 ? g.B0 : g.B1) + (int64_t)(n0 + (row & 127)) * g.ldb + kbeg + ch * 8
                 : g.B0 + (int64_t)(n0 + row) * g.ldb + kbeg + ch * 8;
  }
  auto issue = [&](int kb, int stage) {
    unsigned char* sa = smem + stage * STAGE + (32 * w) * ROWB;
    unsigned char* sb = smem + stage * STAGE + (BM + 32 * w) * ROWB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_global_load_lds(asrc[j] + kb * BK, sa + 8 * j * ROWB, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bsrc[j] + kb * BK, sb + 8 * j * ROWB, 16, 0, 0);
    }
  };

  // operand reads: A rows wm*128 + 32i + lane%32, B rows (per j) from brow_of; K chunk 2s + lane/32
  const int arow = wm * 128 + (lane & 31);
  auto brow_of = [&](int j) {
    return BM + (SW ? j * 128 + wn * 32 : wn * 64 + 32 * j) + (lane & 31);
  };
  int coff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) coff[s] = chunk_pos(2 * s + (lane >> 5), lane & 31) * 16;  // same for all rows used

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) zero(acc[i][j]);

  issue(0, 0);
  if (nkb > 1) issue(1, 1);
  for (int kb = 0; kb < nkb; ++kb) {
    // block kb landed (this wave's 8 loads of block kb + 1 may still be in flight), then every
    // wave's part of it. Plain s_barrier: __syncthreads would also wait for block kb + 1.
    if (kb + 1 < nkb)
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const unsigned char* st = smem + (kb & 1) * STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + (arow + 32 * i) * ROWB + coff[s]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(st + brow_of(j) * ROWB + coff[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave is done with this stage
    if (kb + 2 < nkb) issue(kb + 2, kb & 1);
  }

  if constexpr (EPI == EPI_RMW) {
    // W += alpha * acc through LDS in four passes of 64 rows, so that the fp32 state is read and
    // written in whole 16-byte runs per lane (1 KB per row) with eight loads in flight per thread
    constexpr int LDE = BN + 4;                 // padded fp32 row
    float* ep = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      if (wm == (pass >> 1)) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (pass & 1) + ii;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              ep[(32 * ii + acc_row(r, lane)) * LDE + wn * 64 + 32 * j + acc_col(lane)] = acc[i][j][r];
        }
      }
      __syncthreads();
      f32x4 wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int f = tid + THREADS * q, row = f >> 6, c4 = (f & 63) * 4;
        wv[q] = *reinterpret_cast<const f32x4*>(g.Wf + (int64_t)(m0 + 64 * pass + row) * g.ldw + n0 + c4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int f = tid + THREADS * q, row = f >> 6, c4 = (f & 63) * 4;
        const f32x4 a = *reinterpret_cast<const f32x4*>(ep + row * LDE + c4);
        const f32x4 v = wv[q] + g.alpha * a;
        const int64_t idx = (int64_t)(m0 + 64 * pass + row) * g.ldw + n0 + c4;
        *reinterpret_cast<f32x4*>(g.Wf + idx) = v;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 s4 = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                           static_cast<__bf16>(v[3])};
        *reinterpret_cast<bf16x4*>(g.Wsh + idx) = s4;
      }
      __syncthreads();
    }
    return;
  }

  // epilogues: tile (i, j) element r at row m0 + wm*128 + 32i + acc_row, column n + acc_col
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mb = m0 + wm * 128 + 32 * i;
    if constexpr (SW) {
      const int n = n0 + wn * 32 + acc_col(lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __bf16 zv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q + e;
          const float gt = acc[i][0][r], up = acc[i][1][r];
          zv[e] = static_cast<__bf16>(gt * sigmoidf_(gt) * up);
          g.C[(int64_t)(mb + acc_row(r, lane)) * g.ldc + n] = zv[e];
        }
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 v4 = {zv[0], zv[1], zv[2], zv[3]};
        *reinterpret_cast<bf16x4*>(g.Ct + (int64_t)n * g.ldct + mb + acc_row(4 * q, lane)) = v4;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + 32 * j + acc_col(lane);
        if constexpr (EPI == EPI_STORE) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            g.C[(int64_t)(mb + acc_row(r, lane)) * g.ldc + n] = static_cast<__bf16>(acc[i][j][r]);
        } else if constexpr (EPI == EPI_PARTIAL) {
          float* pp = part + (int64_t)ks * g.M * g.N;
#pragma unroll
          for (int r = 0; r < 16; ++r) pp[(int64_t)(mb + acc_row(r, lane)) * g.N + n] = acc[i][j][r];
        }
      }
    }
  }
}

// C[m][n] = bf16(sum over splits of part[s][m][n]), splits in order. grid-stride over float4.
__global__ void __launch_bounds__(256) ksplit_sum_kernel(const float* part, int ksplit, int M, int N,
                                                         __bf16* C, int64_t ldc) {
  const int64_t mn = (int64_t)M * N;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += (int64_t)gridDim.x * 1024) {
    f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
    for (int s = 1; s < ksplit; ++s) v += *reinterpret_cast<const f32x4*>(part + s * mn + i);
    const int64_t m = i / N, n = i % N;
    __bf16* d = C + m * ldc + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = static_cast<__bf16>(v[e]);
  }
}

template <int EPI>
inline bool fits(const Args& g) {
  return g.M % BM == 0 && g.N % tile_n<EPI>() == 0 && g.K % BK == 0 && g.K >= BK;
}
// splits of K that bring the grid to about one workgroup per CU, each at least 8 K blocks
inline int choose_ksplit(const Args& g, int tiles) {
  int best = 1;
  for (int s = 2; s <= 16; ++s) {
    if (tiles * (s - 1) >= 256) break;
    if ((g.K / BK) % s == 0 && g.K / BK / s >= 8) best = s;
  }
  return best;
}

// W_down update with two workgroups per CU: 256 x 128 output tiles, 4 waves of 128 x 64, one LDS
// stage of 48 KB (so two workgroups fit), K in blocks of 64. Each workgroup loads, waits and
// computes in turn; the other workgroup on the CU fills the MFMA pipe meanwhile, and one
// workgroup's fp32 read-modify-write epilogue overlaps the other's products.
constexpr int PP_BN = 128;
constexpr int PP_LDS = (BM + PP_BN) * ROWB;  // 48 KB

__global__ void __launch_bounds__(256) gemm_rmw_pp_kernel(Args g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int ntn = g.N / PP_BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * PP_BN;
  const int nkb = g.K / BK;
  // staging: A rows 64w + 8j (j < 8), B rows 32w + 8j (j < 4); lane l: row + l/8, LDS chunk l%8
  const int lr = lane >> 3;
  auto issue = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 64 * w + 8 * j + lr;
      __builtin_amdgcn_global_load_lds(g.A + (int64_t)(m0 + row) * g.lda + kb * BK + chunk_pos(lane & 7, row) * 8,
                                       smem + (64 * w + 8 * j) * ROWB, 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 32 * w + 8 * j + lr;
      __builtin_amdgcn_global_load_lds(g.B0 + (int64_t)(n0 + row) * g.ldb + kb * BK + chunk_pos(lane & 7, row) * 8,
                                       smem + (BM + 32 * w + 8 * j) * ROWB, 16, 0, 0);
    }
  };
  const int arow = wm * 128 + (lane & 31), brow = BM + wn * 64 + (lane & 31);
  int coff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) coff[s] = chunk_pos(2 * s + (lane >> 5), lane & 31) * 16;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) zero(acc[i][j]);
  // fp32 state rows of pass p (64 rows x 128 columns, 8 float4 per thread), requested ahead
  const int tid = threadIdx.x;
  auto loadw = [&](int pass, f32x4 (&wv)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int f = tid + 256 * q, row = f >> 5, c4 = (f & 31) * 4;
      wv[q] = *reinterpret_cast<const f32x4*>(g.Wf + (int64_t)(m0 + 64 * pass + row) * g.ldw + n0 + c4);
    }
  };
  f32x4 wv[8];
  for (int kb = 0; kb < nkb; ++kb) {
    issue(kb);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (kb == nkb - 1) loadw(0, wv);  // in flight during the last block's products
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(smem + (arow + 32 * i) * ROWB + coff[s]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(smem + (brow + 32 * j) * ROWB + coff[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the stage is reloaded next
  }
  // W += alpha * acc through LDS in four passes of 64 rows (16-byte runs of the fp32 state); the
  // state rows of pass p + 1 are requested as soon as pass p has consumed its own
  constexpr int LDE = PP_BN + 4;
  float* ep = reinterpret_cast<float*>(smem);
  auto pass_rmw = [&](int pass) {
    if (wm == (pass >> 1)) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * (pass & 1) + ii;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ep[(32 * ii + acc_row(r, lane)) * LDE + wn * 64 + 32 * j + acc_col(lane)] = acc[i][j][r];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // (the state requests stay in flight)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int f = tid + 256 * q, row = f >> 5, c4 = (f & 31) * 4;
      const f32x4 a = *reinterpret_cast<const f32x4*>(ep + row * LDE + c4);
      const f32x4 v = wv[q] + g.alpha * a;
      const int64_t idx = (int64_t)(m0 + 64 * pass + row) * g.ldw + n0 + c4;
      *reinterpret_cast<f32x4*>(g.Wf + idx) = v;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 s4 = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                         static_cast<__bf16>(v[3])};
      *reinterpret_cast<bf16x4*>(g.Wsh + idx) = s4;
    }
    if (pass + 1 < 4) loadw(pass + 1, wv);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the staging area is rewritten next
  };
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) pass_rmw(pass);
}
}  // namespace gemm2

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

// Helper stream and events of the In-Place path, one set per device, created on first use and
// kept for the life of the process. The stream has the default priority.
struct InplaceStreams {
  hipStream_t zs = nullptr;
  hipEvent_t start = nullptr, zdone[2] = {nullptr, nullptr}, zfree[2] = {nullptr, nullptr};
};
static hipError_t inplace_streams(InplaceStreams** out) {
  static std::mutex mu;
  static InplaceStreams sets[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  InplaceStreams& s = sets[dev];
  if (!s.zs) {
    InplaceStreams t;
    e = hipStreamCreateWithFlags(&t.zs, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t.start, hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&t.zdone[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&t.zfree[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) return e;
    s = t;
  }
  *out = &s;
  return hipSuccess;
}

// One TN GEMM: the large-tile kernel where the shape fits its tile, else the 128 x 128 kernel.
// EPI_STORE with ksplit > 1 goes through fp32 partials in `part` and the split sum.
template <int EPI>
static hipError_t run_gemm(const gemm::Args& g, int ksplit, float* part, hipStream_t st) {
  if (EPI == gemm::EPI_RMW && g.M % gemm2::BM == 0 && g.N % gemm2::PP_BN == 0 && g.K % gemm2::BK == 0 &&
      g.K >= gemm2::BK) {
    const unsigned tiles = (unsigned)((g.M / gemm2::BM) * (g.N / gemm2::PP_BN));
    hipLaunchKernelGGL(gemm2::gemm_rmw_pp_kernel, dim3(tiles), dim3(256), gemm2::PP_LDS, st, g);
    return hipGetLastError();
  }
  if (gemm2::fits<EPI>(g)) {
    const unsigned tiles = (unsigned)((g.M / gemm2::BM) * (g.N / gemm2::tile_n<EPI>()));
    if (EPI == gemm::EPI_STORE && ksplit > 1) {
      hipLaunchKernelGGL(gemm2::gemm_big_kernel<gemm2::EPI_PARTIAL>, dim3(tiles * ksplit), dim3(gemm2::THREADS),
                         gemm2::LDS, st, g, ksplit, part);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(gemm2::ksplit_sum_kernel, dim3(1024), dim3(256), 0, st, part, ksplit, g.M, g.N, g.C, g.ldc);
    } else {
      hipLaunchKernelGGL(gemm2::gemm_big_kernel<EPI>, dim3(tiles), dim3(gemm2::THREADS), gemm2::LDS, st, g, 1, part);
    }
  } else {
    const dim3 grid((unsigned)(g.N / gemm::BN), (unsigned)(g.M / gemm::BM));
    hipLaunchKernelGGL(gemm::gemm_tn_kernel<EPI>, grid, dim3(256), gemm::lds_bytes<EPI>(), st, g);
  }
  return hipGetLastError();
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
  // GEMM shapes of one chunk: Z [C x d_H] (K d), apply [C x d] (K d_H), update [d x d_H] (K C)
  gemm::Args za{}, aa{}, ua{};
  za.M = q.chunk, za.N = q.d_hidden, za.K = q.d_model;
  aa.M = q.chunk, aa.N = q.d_model, aa.K = q.d_hidden;
  ua.M = q.d_model, ua.N = q.d_hidden, ua.K = q.chunk;
  const int ks_apply =
      gemm2::fits<EPI_STORE>(aa)
          ? gemm2::choose_ksplit(aa, (aa.M / gemm2::BM) * (aa.N / gemm2::tile_n<EPI_STORE>()))
          : 1;
  WorkspacePlan plan;
  const size_t oWf = plan.add(W_down_out ? 0 : (size_t)nW * 4);
  const size_t oPart = plan.add(ks_apply > 1 ? (size_t)ks_apply * q.chunk * q.d_model * 4 : 0);
  const size_t oSh = plan.add((size_t)nW * 2);
  const size_t oVt = plan.add((size_t)q.d_model * q.N * 2);
  // Z and Z^T double-buffered: chunk i + 1's Z is produced while chunk i is applied and written
  const size_t oZ = plan.add((size_t)2 * q.chunk * q.d_hidden * 2);
  const size_t oZt = plan.add((size_t)2 * q.chunk * q.d_hidden * 2);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  __bf16* Wsh = reinterpret_cast<__bf16*>(ws + oSh);
  __bf16* Vt = reinterpret_cast<__bf16*>(ws + oVt);
  __bf16* Zb[2] = {reinterpret_cast<__bf16*>(ws + oZ), reinterpret_cast<__bf16*>(ws + oZ) + (int64_t)q.chunk * q.d_hidden};
  __bf16* Ztb[2] = {reinterpret_cast<__bf16*>(ws + oZt),
                    reinterpret_cast<__bf16*>(ws + oZt) + (int64_t)q.chunk * q.d_hidden};
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(gemm_tn_kernel<EPI_SWIGLU>, lds_bytes<EPI_SWIGLU>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_STORE>, lds_bytes<EPI_STORE>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_RMW>, lds_bytes<EPI_RMW>());
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_SWIGLU>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_STORE>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_RMW>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_rmw_pp_kernel, gemm2::PP_LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<gemm2::EPI_PARTIAL>, gemm2::LDS);
    return e;
  }();
  float* part = reinterpret_cast<float*>(ws + oPart);
  TTT_HIP(lds_ok);
  const __bf16* Hb = static_cast<const __bf16*>(Hs);
  const __bf16* Vb = static_cast<const __bf16*>(Vbar);
  __bf16* Ob = static_cast<__bf16*>(O);
  const int nch = q.N / q.chunk;
  // Z depends only on the inputs and W_gate / W_up, so it runs on a helper stream: Z of chunk i
  // into buffer i % 2 after the chunk that last read that buffer was written (event zfree), and
  // the caller's stream waits for it (event zdone) before the chunk's apply.
  InplaceStreams* hs = nullptr;
  TTT_HIP(inplace_streams(&hs));
  hipStream_t zs = hs->zs;
  TTT_HIP(hipEventRecord(hs->start, st));
  TTT_HIP(hipStreamWaitEvent(zs, hs->start, 0));
  bool freed[2] = {false, false};
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
      const int zb = i & 1;
      __bf16* Z = Zb[zb];
      __bf16* Zt = Ztb[zb];
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
      if (freed[zb]) TTT_HIP(hipStreamWaitEvent(zs, hs->zfree[zb], 0));
      {
        LaunchTimer lt(K_INP_Z, zs);
        TTT_HIP(run_gemm<EPI_SWIGLU>(z, 1, part, zs));
      }
      TTT_HIP(hipEventRecord(hs->zdone[zb], zs));
      TTT_HIP(hipStreamWaitEvent(st, hs->zdone[zb], 0));
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
        TTT_HIP(run_gemm<EPI_STORE>(a, ks_apply, part, st));
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
        TTT_HIP(run_gemm<EPI_RMW>(u, 1, part, st));
      }
      TTT_HIP(hipEventRecord(hs->zfree[zb], st));
      freed[zb] = true;
    }
  }
  return TTT_OK;
}
