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
enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_RMW = 2, EPI_SWIGLU_BWD = 4 };

struct Args {
  const __bf16* A;  int64_t lda;    // [M][K]
  const __bf16* B0; int64_t ldb;    // [N][K]
  const __bf16* B1;                 // second B (SwiGLU up projection)
  int M, N, K;
  __bf16* C; int64_t ldc;           // STORE / SWIGLU row-major output [M][N]
  __bf16* Ct; int64_t ldct;         // SWIGLU transposed output [N][M]
  float* Wf; __bf16* Wsh; int64_t ldw;  // RMW state and shadow [M][N]
  float alpha;
  // Concatenated K (K1 > 0): K blocks k >= K1 read A2 / B2 at k - K1 (same leading dimensions),
  // so C = A B^T + A2 B2^T in one product.
  const __bf16* A2; const __bf16* B2; int K1;
  // SWIGLU: when Ga is set, the gate and up products are also stored (bf16, [M][N], ld ldc).
  // SWIGLU_BWD: the accumulator is dZ; Ga / Gu hold the stored gate and up products, and the
  // outputs are dA (C, Ct) and dU (C2, Ct2), row-major [M][N] (ld ldc) and transposed (ld ldct).
  __bf16* Ga; __bf16* Gu;
  __bf16* C2; __bf16* Ct2;
  // RMW of the two-workgroups-per-CU kernel only: the shadow is bf16(shscale * W) (0 means 1),
  // Wsh may be null, and Wsht (if set) receives the shadow transposed ([N][M], ld ldwt).
  float shscale;
  __bf16* Wsht; int64_t ldwt;
};

// operand base of the K block starting at k (concatenated-K products switch at K1)
__device__ __forceinline__ const __bf16* a_at(const Args& g, int k) {
  return (g.K1 > 0 && k >= g.K1) ? g.A2 + (k - g.K1) : g.A + k;
}
__device__ __forceinline__ const __bf16* b_at(const Args& g, int k) {
  return (g.K1 > 0 && k >= g.K1) ? g.B2 + (k - g.K1) : g.B0 + k;
}

// dA = dZ * U * silu'(A), dU = dZ * silu(A) for the gate product a and the up product u
__device__ __forceinline__ void swiglu_bwd(float dz, float a, float u, float& da, float& du) {
  const float sg = sigmoidf_(a);
  da = dz * u * (sg * (1.f + a * (1.f - sg)));
  du = dz * a * sg;
}

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
    const __bf16* Ab = a_at(g, k0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ra[v] = *reinterpret_cast<const u32x4*>(Ab + (int64_t)(m0 + lr + 32 * v) * g.lda + lc);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const __bf16* Bp = b == 0 ? b_at(g, k0) : g.B1 + k0;
        rb[b][v] = *reinterpret_cast<const u32x4*>(Bp + (int64_t)(n0 + lr + 32 * v) * g.ldb + lc);
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
            const int64_t o = (int64_t)(mb + acc_row(r, lane)) * g.ldc + n;
            g.C[o] = zv[e];
            if (g.Ga) {
              g.Ga[o] = static_cast<__bf16>(gt);
              g.Gu[o] = static_cast<__bf16>(up);
            }
          }
          // 4 consecutive rows m -> 4 consecutive elements of row n of the transposed copy
          __bf16* dst = g.Ct + (int64_t)n * g.ldct + mb + acc_row(4 * q, lane);
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v4 = {zv[0], zv[1], zv[2], zv[3]};
          *reinterpret_cast<bf16x4*>(dst) = v4;
        }
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __bf16 da[4], du[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            const int64_t o = (int64_t)(mb + acc_row(r, lane)) * g.ldc + n;
            float fa, fu;
            swiglu_bwd(acc[0][i][j][r], static_cast<float>(g.Ga[o]), static_cast<float>(g.Gu[o]), fa, fu);
            da[e] = static_cast<__bf16>(fa);
            du[e] = static_cast<__bf16>(fu);
            g.C[o] = da[e];
            g.C2[o] = du[e];
          }
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const int64_t to = (int64_t)n * g.ldct + mb + acc_row(4 * q, lane);
          *reinterpret_cast<bf16x4*>(g.Ct + to) = bf16x4{da[0], da[1], da[2], da[3]};
          *reinterpret_cast<bf16x4*>(g.Ct2 + to) = bf16x4{du[0], du[1], du[2], du[3]};
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
constexpr int BWD_LDR = BN + 8;                 // SwiGLU-backward epilogue: padded bf16 row
constexpr int BWD_LDS = 4 * 64 * BWD_LDR * 2;   // its four staged 64-row tiles (132 KB)
template <int EPI>
constexpr int lds_of() { return EPI == gemm::EPI_SWIGLU_BWD && BWD_LDS > LDS ? BWD_LDS : LDS; }
constexpr int EPI_PARTIAL = 3;                  // fp32 partial of one K split

template <int EPI>
constexpr int tile_n() { return EPI == EPI_SWIGLU ? BN / 2 : BN; }

__device__ __forceinline__ int chunk_pos(int c, int row) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

// grid: ksplit * (M / BM) * (N / tile_n) workgroups of 512 threads; split fastest, then N tile.
// Wave w: rows (w & 1) * 128.. of the A tile; B rows (w >> 1) * 64.. (SwiGLU: gate rows
// (w >> 1) * 32.. and the same up rows, so each wave holds both factors of its outputs).
template <int EPI>
__device__ __forceinline__ void gemm_big_body(const Args& g, int ksplit, float* part, int bid, unsigned char* smem) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int TN = tile_n<EPI>();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int ntn = g.N / TN;
  const int ks = bid % ksplit;
  bid /= ksplit;
  const int m0 = (bid / ntn) * BM, n0 = (bid % ntn) * TN;
  const int kper = g.K / ksplit, kbeg = ks * kper, nkb = kper / BK;

  // staging: instruction j of wave w fills rows 32w + 8j .. +8 of each operand tile; lane l
  // takes row + l/8 and LDS chunk l%8
  const int lr = lane >> 3;
  int64_t aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * w + 8 * j + lr;
    const int ch = chunk_pos(lane & 7, row);
    aoff[j] = (int64_t)(m0 + row) * g.lda + ch * 8;
    // B tile rows: SwiGLU rows 0..127 gate, 128..255 up (same hidden units n0..n0+127)
    boff[j] = (int64_t)(n0 + (SW ? (row & 127) : row)) * g.ldb + ch * 8;
  }
  auto issue = [&](int kb, int stage) {
    unsigned char* sa = smem + stage * STAGE + (32 * w) * ROWB;
    unsigned char* sb = smem + stage * STAGE + (BM + 32 * w) * ROWB;
    const int k = kbeg + kb * BK;
    const __bf16* Ab = a_at(g, k);
    // SwiGLU: waves 0-3 stage gate rows, waves 4-7 up rows
    const __bf16* Bb = SW ? (w < 4 ? g.B0 : g.B1) + k : b_at(g, k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_global_load_lds(Ab + aoff[j], sa + 8 * j * ROWB, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Bb + boff[j], sb + 8 * j * ROWB, 16, 0, 0);
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

  if constexpr (EPI == gemm::EPI_SWIGLU_BWD) {
    // dA, dU through LDS in four passes of 64 rows: the stored gate and up products are read and
    // the token-major outputs written in 16-byte runs; the transposed outputs go out from the
    // accumulators (four consecutive rows per lane, 8-byte stores)
    constexpr int LDR = BWD_LDR;
    __bf16* gaS = reinterpret_cast<__bf16*>(smem);  // [64][LDR] each
    __bf16* guS = gaS + 64 * LDR;
    __bf16* daS = guS + 64 * LDR;
    __bf16* duS = daS + 64 * LDR;
    const int tid = threadIdx.x;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int r0 = m0 + 64 * pass;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = tid + THREADS * q, row = f >> 5, c8 = (f & 31) * 8;
        const int64_t o = (int64_t)(r0 + row) * g.ldc + n0 + c8;
        *reinterpret_cast<u32x4*>(gaS + row * LDR + c8) = *reinterpret_cast<const u32x4*>(g.Ga + o);
        *reinterpret_cast<u32x4*>(guS + row * LDR + c8) = *reinterpret_cast<const u32x4*>(g.Gu + o);
      }
      __syncthreads();
      if (wm == (pass >> 1)) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (pass & 1) + ii;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int cl = wn * 64 + 32 * j + acc_col(lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              __bf16 da[4], du[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * q + e, lo = (32 * ii + acc_row(r, lane)) * LDR + cl;
                float fa, fu;
                gemm::swiglu_bwd(acc[i][j][r], static_cast<float>(gaS[lo]), static_cast<float>(guS[lo]), fa, fu);
                da[e] = static_cast<__bf16>(fa);
                du[e] = static_cast<__bf16>(fu);
                daS[lo] = da[e];
                duS[lo] = du[e];
              }
              const int64_t to = (int64_t)(n0 + cl) * g.ldct + r0 + 32 * ii + acc_row(4 * q, lane);
              *reinterpret_cast<bf16x4*>(g.Ct + to) = bf16x4{da[0], da[1], da[2], da[3]};
              *reinterpret_cast<bf16x4*>(g.Ct2 + to) = bf16x4{du[0], du[1], du[2], du[3]};
            }
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = tid + THREADS * q, row = f >> 5, c8 = (f & 31) * 8;
        const int64_t o = (int64_t)(r0 + row) * g.ldc + n0 + c8;
        *reinterpret_cast<u32x4*>(g.C + o) = *reinterpret_cast<const u32x4*>(daS + row * LDR + c8);
        *reinterpret_cast<u32x4*>(g.C2 + o) = *reinterpret_cast<const u32x4*>(duS + row * LDR + c8);
      }
      __syncthreads();  // the staging tiles are rewritten by the next pass
    }
    return;
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
        if (g.Wsh) *reinterpret_cast<bf16x4*>(g.Wsh + idx) = s4;
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
          const int64_t o = (int64_t)(mb + acc_row(r, lane)) * g.ldc + n;
          g.C[o] = zv[e];
          if (g.Ga) {
            g.Ga[o] = static_cast<__bf16>(gt);
            g.Gu[o] = static_cast<__bf16>(up);
          }
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

template <int EPI>
__global__ void __launch_bounds__(512) gemm_big_kernel(Args g, int ksplit, float* part) {
  extern __shared__ __align__(16) unsigned char smem[];
  gemm_big_body<EPI>(g, ksplit, part, blockIdx.x, smem);
}

// Two independent products in one launch: the first nfirst workgroups form product g1 (epilogue
// E1, no K split), the others product g2 (epilogue E2, ksplit-way K split into part). Used to
// produce the next chunk's Z beside the current chunk's apply on the caller's stream.
template <int E1, int E2>
__global__ void __launch_bounds__(512) gemm_big_pair_kernel(Args g1, int nfirst, Args g2, int ksplit, float* part) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < nfirst)
    gemm_big_body<E1>(g1, 1, part, blockIdx.x, smem);
  else
    gemm_big_body<E2>(g2, ksplit, part, blockIdx.x - nfirst, smem);
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
constexpr int PP_LDE = PP_BN + 4;            // padded fp32 row of the epilogue tile
constexpr int PP_LDT = 64 + 2;               // transposed-shadow tile row (bf16)
// with a transposed shadow: the epilogue tile, then the transposed bf16 tile [128][PP_LDT]
constexpr int PP_LDS_T = 64 * PP_LDE * 4 + PP_BN * PP_LDT * 2;
static_assert(PP_LDS_T <= 80 * 1024, "two workgroups per CU");

// TSH: also the scaled and transposed shadows (Args::shscale, Args::Wsht); Wsh may be null.
template <bool TSH>
__global__ void __launch_bounds__(256, 2) gemm_rmw_pp_kernel(Args g) {
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
  constexpr int LDE = PP_LDE;
  float* ep = reinterpret_cast<float*>(smem);
  __bf16* tp = reinterpret_cast<__bf16*>(smem + 64 * LDE * 4);  // [PP_BN][PP_LDT] transposed shadow
  const float shs = !TSH || g.shscale == 0.f ? 1.f : g.shscale;
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
      const bf16x4 s4 = {static_cast<__bf16>(shs * v[0]), static_cast<__bf16>(shs * v[1]),
                         static_cast<__bf16>(shs * v[2]), static_cast<__bf16>(shs * v[3])};
      if (!TSH || g.Wsh) *reinterpret_cast<bf16x4*>(g.Wsh + idx) = s4;
      if (TSH && g.Wsht) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tp[(c4 + e) * PP_LDT + row] = s4[e];
      }
    }
    if (pass + 1 < 4) loadw(pass + 1, wv);
    if (TSH && g.Wsht) {  // the pass's 64 x 128 shadow tile, transposed: 128 rows of 64 bf16, 16 bytes per store
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = tid + 256 * q, n = f >> 3, m8 = (f & 7) * 8;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(tp + n * PP_LDT + m8);  // 4-byte aligned rows
        const u32x4 v = {src[0], src[1], src[2], src[3]};
        *reinterpret_cast<u32x4*>(g.Wsht + (int64_t)(n0 + n) * g.ldwt + m0 + 64 * pass + m8) = v;
      }
    }
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

// LM-aligned target of one sequence: C[t][c] = sum_{tau < k} taps[tau][c] * X0[t + tau][c] (zero
// past row N - 1), accumulated in float32 and rounded to bf16. TRANS writes C^T [dm][N] (the
// layout the update reads Vbar in), else C [N][dm]. grid (dm / 64, N / 64), block 256: a 64 x 64
// output tile from a (64 + k - 1) x 64 window of X0 staged in LDS.
template <bool TRANS>
__global__ void __launch_bounds__(256) target_conv_kernel(const __bf16* __restrict__ X0, const float* __restrict__ taps,
                                                         int k, int N, int dm, __bf16* __restrict__ out) {
  __shared__ float win[64 + 15][65];
  __shared__ float tp[16][64];
  const int c0 = blockIdx.x * 64, t0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int i = tid; i < (64 + k - 1) * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    win[r][c] = t0 + r < N ? static_cast<float>(X0[(int64_t)(t0 + r) * dm + c0 + c]) : 0.f;
  }
  for (int i = tid; i < k * 64; i += 256) tp[i / 64][i % 64] = taps[(int64_t)(i / 64) * dm + c0 + i % 64];
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    // TRANS: consecutive threads take consecutive tokens of one channel (coalesced along N)
    const int r = TRANS ? i % 64 : i / 64, c = TRANS ? i / 64 : i % 64;
    float acc = 0.f;
    for (int tau = 0; tau < k; ++tau) acc = fmaf(tp[tau][c], win[r + tau][c], acc);
    const __bf16 v = static_cast<__bf16>(acc);
    if (TRANS)
      out[(int64_t)(c0 + c) * N + t0 + r] = v;
    else
      out[(int64_t)(t0 + r) * dm + c0 + c] = v;
  }
}

// [R][C] float32 -> [C][R] float32 and its bf16 copy, through a 64 x 64 LDS tile.
// grid (C / 64, R / 64), block 256.
__global__ void __launch_bounds__(256) transpose_f32_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                           __bf16* __restrict__ dsh, int R, int C) {
  __shared__ float t[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) t[i / 64][i % 64] = src[(int64_t)(r0 + i / 64) * C + c0 + i % 64];
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const float v = t[i % 64][i / 64];
    const int64_t o = (int64_t)(c0 + i / 64) * R + r0 + i % 64;
    dst[o] = v;
    dsh[o] = static_cast<__bf16>(v);
  }
}

// dst[i] = 0 (add == 0) or dst[i] += src[i] (add == 1) over n floats. grid-stride.
__global__ void __launch_bounds__(256) f32_zero_add_kernel(float* dst, const float* src, int64_t n, int add) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = add ? dst[i] + src[i] : 0.f;
}

// One TN GEMM: the large-tile kernel where the shape fits its tile, else the 128 x 128 kernel.
// EPI_STORE with ksplit > 1 goes through fp32 partials in `part` and the split sum.
template <int EPI>
static hipError_t run_gemm(int cls, const gemm::Args& g, int ksplit, float* part, hipStream_t st) {
  if (EPI == gemm::EPI_RMW && g.M % gemm2::BM == 0 && g.N % gemm2::PP_BN == 0 && g.K % gemm2::BK == 0 &&
      g.K >= gemm2::BK) {
    const unsigned tiles = (unsigned)((g.M / gemm2::BM) * (g.N / gemm2::PP_BN));
    return launch_k(cls, gemm2::gemm_rmw_pp_kernel<false>, dim3(tiles), dim3(256), gemm2::PP_LDS, st, g);
  }
  if (gemm2::fits<EPI>(g)) {
    const unsigned tiles = (unsigned)((g.M / gemm2::BM) * (g.N / gemm2::tile_n<EPI>()));
    if (EPI == gemm::EPI_STORE && ksplit > 1) {
      hipError_t e = launch_k(cls, gemm2::gemm_big_kernel<gemm2::EPI_PARTIAL>, dim3(tiles * ksplit),
                              dim3(gemm2::THREADS), gemm2::LDS, st, g, ksplit, part);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(gemm2::ksplit_sum_kernel, dim3(1024), dim3(256), 0, st, part, ksplit, g.M, g.N, g.C, g.ldc);
      return hipGetLastError();
    }
    return launch_k(cls, gemm2::gemm_big_kernel<EPI>, dim3(tiles), dim3(gemm2::THREADS), gemm2::lds_of<EPI>(), st, g,
                    1, part);
  }
  const dim3 grid((unsigned)(g.N / gemm::BN), (unsigned)(g.M / gemm::BM));
  return launch_k(cls, gemm::gemm_tn_kernel<EPI>, grid, dim3(256), gemm::lds_bytes<EPI>(), st, g);
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
  const bool target = q.X0 != nullptr;  // the LM-aligned target is built here
  if (target && (Vbar || !q.conv_taps || q.conv_k < 1 || q.conv_k > 16)) return TTT_ERR_ARG;
  if (q.B > 0 && !W_down) return TTT_ERR_ARG;
  if (q.B > 0 && q.N > 0 && (!Hs || !W_gate || !W_up || (!Vbar && !target) || !O)) return TTT_ERR_ARG;
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
  const size_t oC = plan.add(target && q.W_target ? (size_t)q.N * q.d_model * 2 : 0);  // Conv1D(X0) before W_target
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
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_rmw_pp_kernel<false>, gemm2::PP_LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<gemm2::EPI_PARTIAL>, gemm2::LDS);
    return e;
  }();
  float* part = reinterpret_cast<float*>(ws + oPart);
  TTT_HIP(lds_ok);
  const __bf16* Hb = static_cast<const __bf16*>(Hs);
  const __bf16* Vb = static_cast<const __bf16*>(Vbar);
  __bf16* Ob = static_cast<__bf16*>(O);
  const int nch = q.N / q.chunk;
  // Z of a chunk depends only on H and W_gate / W_up. Where both products take the large-tile
  // kernel, chunk i + 1's Z (into buffer (i + 1) % 2, whose last readers -- chunk i - 1's apply
  // and update -- came earlier on the stream) is formed in the same launch as chunk i's apply, so
  // the two fill the chip together; everything runs on the caller's stream.
  const bool paired = gemm2::fits<EPI_SWIGLU>(za) && gemm2::fits<EPI_STORE>(aa) && ks_apply > 1;
  const unsigned ztiles = (unsigned)((za.M / gemm2::BM) * (za.N / gemm2::tile_n<EPI_SWIGLU>()));
  const unsigned atiles = (unsigned)((aa.M / gemm2::BM) * (aa.N / gemm2::tile_n<EPI_STORE>())) * (unsigned)ks_apply;
  if (paired) TTT_HIP(allow_lds(gemm2::gemm_big_pair_kernel<EPI_SWIGLU, gemm2::EPI_PARTIAL>, gemm2::LDS));
  for (int b = 0; b < q.B; ++b) {
    float* Wf = W_down_out ? W_down_out + (int64_t)b * nW : reinterpret_cast<float*>(ws + oWf);
    TTT_HIP(hipMemcpyAsync(Wf, W_down + (int64_t)b * q.wdown_batch_stride, (size_t)nW * 4,
                           hipMemcpyDeviceToDevice, st));
    if (nch == 0) continue;
    {
      LaunchTimer lt(K_INP_PREP, st);
      hipLaunchKernelGGL(to_bf16_kernel, dim3(2048), dim3(256), 0, st, Wf, Wsh, nW);
      TTT_HIP(hipGetLastError());
      if (!target) {
        hipLaunchKernelGGL(transpose_bf16_kernel, dim3(q.d_model / 64, q.N / 64), dim3(256), 0, st,
                           Vb + (int64_t)b * q.N * q.d_model, Vt, q.N, q.d_model);
        TTT_HIP(hipGetLastError());
      }
    }
    if (target) {
      // Vbar^T [d_model][N]: the convolution written transposed, or its row-major result C
      // through Vbar^T = W_target C^T (a TN product: A = W_target [out][in], B = C [N][in])
      const __bf16* X0b = static_cast<const __bf16*>(q.X0) + (int64_t)b * q.N * q.d_model;
      const dim3 cgrid((unsigned)(q.d_model / 64), (unsigned)(q.N / 64));
      if (!q.W_target) {
        LaunchTimer lt(K_INP_PREP, st);
        hipLaunchKernelGGL(target_conv_kernel<true>, cgrid, dim3(256), 0, st, X0b, q.conv_taps, q.conv_k, q.N,
                           q.d_model, Vt);
        TTT_HIP(hipGetLastError());
      } else {
        __bf16* Cb = reinterpret_cast<__bf16*>(ws + oC);
        {
          LaunchTimer lt(K_INP_PREP, st);
          hipLaunchKernelGGL(target_conv_kernel<false>, cgrid, dim3(256), 0, st, X0b, q.conv_taps, q.conv_k, q.N,
                             q.d_model, Cb);
          TTT_HIP(hipGetLastError());
        }
        Args t{};
        t.A = static_cast<const __bf16*>(q.W_target);
        t.lda = q.d_model;
        t.B0 = Cb;
        t.ldb = q.d_model;
        t.M = q.d_model;
        t.N = q.N;
        t.K = q.d_model;
        t.C = Vt;
        t.ldc = q.N;
        TTT_HIP(run_gemm<EPI_STORE>(K_INP_PREP, t, 1, part, st));
      }
    }
    auto zargs = [&](int i) {
      Args z{};
      z.A = Hb + ((int64_t)b * q.N + (int64_t)i * q.chunk) * q.d_model;
      z.lda = q.d_model;
      z.B0 = static_cast<const __bf16*>(W_gate);
      z.B1 = static_cast<const __bf16*>(W_up);
      z.ldb = q.d_model;
      z.M = q.chunk;
      z.N = q.d_hidden;
      z.K = q.d_model;
      z.C = Zb[i & 1];
      z.ldc = q.d_hidden;
      z.Ct = Ztb[i & 1];
      z.ldct = q.chunk;
      return z;
    };
    if (paired) TTT_HIP(run_gemm<EPI_SWIGLU>(K_INP_Z, zargs(0), 1, part, st));
    for (int i = 0; i < nch; ++i) {
      const int64_t t0 = (int64_t)i * q.chunk;
      const int zb = i & 1;
      Args a{};
      a.A = Zb[zb];
      a.lda = q.d_hidden;
      a.B0 = Wsh;
      a.ldb = q.d_hidden;
      a.M = q.chunk;
      a.N = q.d_model;
      a.K = q.d_hidden;
      a.C = Ob + ((int64_t)b * q.N + t0) * q.d_model;
      a.ldc = q.d_model;
      if (paired) {
        // apply of chunk i (K-split partials) with the Z of chunk i + 1, then the split sum
        const bool next = i + 1 < nch;
        const Args zn = next ? zargs(i + 1) : Args{};
        TTT_HIP(launch_k(next ? K_INP_APPLY_Z : K_INP_APPLY, gemm2::gemm_big_pair_kernel<EPI_SWIGLU, gemm2::EPI_PARTIAL>,
                         dim3((next ? ztiles : 0u) + atiles), dim3(gemm2::THREADS), gemm2::LDS, st, zn,
                         (int)(next ? ztiles : 0u), a, ks_apply, part));
        hipLaunchKernelGGL(gemm2::ksplit_sum_kernel, dim3(1024), dim3(256), 0, st, part, ks_apply, a.M, a.N, a.C,
                           a.ldc);
        TTT_HIP(hipGetLastError());
      } else {
        TTT_HIP(run_gemm<EPI_SWIGLU>(K_INP_Z, zargs(i), 1, part, st));
        TTT_HIP(run_gemm<EPI_STORE>(K_INP_APPLY, a, ks_apply, part, st));
      }
      Args u{};
      u.A = Vt + t0;
      u.lda = q.N;
      u.B0 = Ztb[zb];
      u.ldb = q.chunk;
      u.M = q.d_model;
      u.N = q.d_hidden;
      u.K = q.chunk;
      u.Wf = Wf;
      u.Wsh = Wsh;
      u.ldw = q.d_hidden;
      u.alpha = q.eta;
      TTT_HIP(run_gemm<EPI_RMW>(K_INP_UPDATE, u, 1, part, st));
    }
  }
  return TTT_OK;
}

// ---------------------------------------------------------------------------------------------
// Backward of the In-Place update, per sequence in two sweeps over the chunks, every product a TN
// GEMM of the kernels above. With G_i = dO_i^T Z_i and R_i = sum_{k > i} G_k:
//   dZ_i = dO_i W_i + eta Vbar_i R_i,  dVbar_i = eta Z_i R_i^T,  dW_down = sum_i G_i,
//   dA = dZ * U * silu'(A), dU = dZ * silu(A),  dH_i = dA W_gate + dU W_up,
//   dW_gate = sum_i dA_i^T H_i,  dW_up = sum_i dU_i^T H_i.
// Forward sweep: Z_i (token-major and transposed), the gate and up products A_i, U_i and the
// transposed states W_i^T (bf16) are kept. Reverse sweep per chunk: dZ_i as one product over the
// concatenated K [dO_i | Vbar_i] x [W_i^T | eta R^T]^T whose epilogue applies the SwiGLU backward
// to the stored A_i, U_i and writes dA, dU token-major and transposed (the transposed copies of all
// chunks are kept); dVbar_i against the bf16 shadow of eta R (K split); R += dO_i^T Z_i in fp32
// with both bf16 shadows (eta R and eta R^T, the transposed one from the epilogue); dH_i over the
// concatenated K [dA | dU] x [W_gate^T | W_up^T]^T (K split). After the sweep, dW_gate and dW_up are
// one product each over all tokens of the sequence (K = N), accumulated in fp32 over sequences.
extern "C" ttt_status ttt_inplace_down_backward(const ttt_inplace_params* p, const void* Hs, const void* W_gate,
                                                const void* W_up, const float* W_down, const void* Vbar,
                                                const void* dO, void* dHs, float* dW_gate, float* dW_up,
                                                float* dW_down, void* dVbar, void* workspace,
                                                size_t* workspace_bytes, void* stream) {
  using namespace gemm;
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_inplace_params& q = *p;
  if (q.B < 0 || q.N < 0 || q.d_model <= 0 || q.d_hidden <= 0 || q.chunk <= 0) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (q.wdown_batch_stride < 0) return TTT_ERR_ARG;
  if (q.dtype != TTT_BF16 || q.X0) return TTT_ERR_UNSUPPORTED;  // a device-built target has no backward here
  if (q.N % q.chunk) return TTT_ERR_SHAPE;
  if (q.d_model % 256 || q.d_hidden % 256 || q.chunk % 128) return TTT_ERR_SHAPE;
  const int64_t dm = q.d_model, dh = q.d_hidden, C = q.chunk, N = q.N, nW = dm * dh;
  if (q.wdown_batch_stride != 0 && q.wdown_batch_stride != nW) return TTT_ERR_SHAPE;
  if (q.B > 0 && (!W_down || !dW_down || !dW_gate || !dW_up)) return TTT_ERR_ARG;
  if (q.B > 0 && N > 0 && (!Hs || !W_gate || !W_up || !Vbar || !dO || !dHs || !dVbar)) return TTT_ERR_ARG;
  const int nch = (int)(N / C);
  // K splits of the two token-major products whose K is d_hidden-long (dVbar: K = d_hidden, dH:
  // K = 2 d_hidden), chosen as for the forward's apply
  auto ks_of = [&](int64_t K) {
    Args t{};
    t.M = (int)C;
    t.N = (int)dm;
    t.K = (int)K;
    if (!gemm2::fits<EPI_STORE>(t)) return 1;
    return gemm2::choose_ksplit(t, (int)((C / gemm2::BM) * (dm / gemm2::BN)));
  };
  const int ks_dv = ks_of(dh), ks_dh = ks_of(2 * dh);
  WorkspacePlan plan;
  const size_t oZ = plan.add((size_t)N * dh * 2), oZt = plan.add((size_t)N * dh * 2);  // per chunk [C][dh], [dh][C]
  const size_t oGa = plan.add((size_t)N * dh * 2), oGu = plan.add((size_t)N * dh * 2);
  const size_t oWtSh = plan.add((size_t)nch * nW * 2), oWt = plan.add((size_t)nW * 4);
  const size_t oR = plan.add((size_t)nW * 4), oRsh = plan.add((size_t)nW * 2), oRtsh = plan.add((size_t)nW * 2);
  const size_t odA = plan.add((size_t)C * dh * 2), odU = plan.add((size_t)C * dh * 2);
  const size_t odAt = plan.add((size_t)dh * N * 2), odUt = plan.add((size_t)dh * N * 2);  // [dh][N]
  const size_t oPart = plan.add((size_t)std::max(ks_dv, ks_dh) * C * dm * 4);
  const size_t oVt = plan.add((size_t)dm * N * 2), odOt = plan.add((size_t)dm * N * 2), oHt = plan.add((size_t)dm * N * 2);
  const size_t oWgT = plan.add((size_t)nW * 2), oWuT = plan.add((size_t)nW * 2);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (q.B == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto bfp = [&](size_t o) { return reinterpret_cast<__bf16*>(ws + o); };
  auto f32p = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(gemm_tn_kernel<EPI_SWIGLU>, lds_bytes<EPI_SWIGLU>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_SWIGLU_BWD>, lds_bytes<EPI_SWIGLU_BWD>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_STORE>, lds_bytes<EPI_STORE>());
    if (e == hipSuccess) e = allow_lds(gemm_tn_kernel<EPI_RMW>, lds_bytes<EPI_RMW>());
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_SWIGLU>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_SWIGLU_BWD>, gemm2::lds_of<EPI_SWIGLU_BWD>());
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_STORE>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<gemm2::EPI_PARTIAL>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_rmw_pp_kernel<true>, gemm2::PP_LDS_T);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_rmw_pp_kernel<false>, gemm2::PP_LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_RMW>, gemm2::LDS);
    return e;
  }();
  TTT_HIP(lds_ok);
  const bool shared = q.wdown_batch_stride == 0;
  auto zero = [&](float* d, int64_t n) -> hipError_t {
    hipLaunchKernelGGL(f32_zero_add_kernel, dim3(1024), dim3(256), 0, st, d, static_cast<const float*>(nullptr), n, 0);
    return hipGetLastError();
  };
  // fp32 read-modify-write W += alpha A B^T (two workgroups per CU; every shape here fits it)
  auto rmw = [&](const __bf16* A, int64_t lda, const __bf16* B, int64_t ldb, int64_t M, int64_t Nn, int64_t K, float* Wf,
                 __bf16* Wsh, float alpha, float shs = 1.f, __bf16* Wsht = nullptr,
                 int cls = K_INP_UPDATE) -> hipError_t {
    Args u{};
    u.A = A;
    u.lda = lda;
    u.B0 = B;
    u.ldb = ldb;
    u.M = (int)M;
    u.N = (int)Nn;
    u.K = (int)K;
    u.Wf = Wf;
    u.Wsh = Wsh;
    u.ldw = Nn;
    u.alpha = alpha;
    u.shscale = shs;
    u.Wsht = Wsht;
    u.ldwt = M;
    if (K > 16 * C) {  // a long K (the weight gradients over a whole sequence): the double-buffered kernel
      const unsigned tiles = (unsigned)((M / gemm2::BM) * (Nn / gemm2::BN));
      return launch_k(cls, gemm2::gemm_big_kernel<EPI_RMW>, dim3(tiles), dim3(gemm2::THREADS), gemm2::LDS, st, u, 1,
                      static_cast<float*>(nullptr));
    }
    const unsigned tiles = (unsigned)((M / gemm2::BM) * (Nn / gemm2::PP_BN));
    if (!Wsht && Wsh && shs == 1.f)  // a plain update: the forward's instance (no spills)
      return launch_k(cls, gemm2::gemm_rmw_pp_kernel<false>, dim3(tiles), dim3(256), gemm2::PP_LDS, st, u);
    return launch_k(cls, gemm2::gemm_rmw_pp_kernel<true>, dim3(tiles), dim3(256), gemm2::PP_LDS_T, st, u);
  };
  // bf16 C [M][Nn] = A B^T (+ A2 B2^T over the concatenated K), K-split through fp32 partials
  auto store = [&](const __bf16* A, const __bf16* B, const __bf16* A2, const __bf16* B2, int64_t lda, int64_t K1,
                   int64_t K, int64_t Nn, __bf16* Cout, int ks) -> hipError_t {
    Args t{};
    t.A = A;
    t.lda = lda;
    t.B0 = B;
    t.ldb = lda;
    t.A2 = A2;
    t.B2 = B2;
    t.K1 = (int)K1;
    t.M = (int)C;
    t.N = (int)Nn;
    t.K = (int)K;
    t.C = Cout;
    t.ldc = Nn;
    return run_gemm<EPI_STORE>(K_INP_APPLY, t, ks, f32p(oPart), st);
  };
  const __bf16* Wg = static_cast<const __bf16*>(W_gate);
  const __bf16* Wu = static_cast<const __bf16*>(W_up);
  {
    LaunchTimer lt(K_INP_PREP, st);
    TTT_HIP(zero(dW_gate, nW));
    TTT_HIP(zero(dW_up, nW));
    if (shared) TTT_HIP(zero(dW_down, nW));
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(dm / 64), (unsigned)(dh / 64)), dim3(256), 0, st, Wg,
                       bfp(oWgT), (int)dh, (int)dm);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(dm / 64), (unsigned)(dh / 64)), dim3(256), 0, st, Wu,
                       bfp(oWuT), (int)dh, (int)dm);
    TTT_HIP(hipGetLastError());
  }
  for (int b = 0; b < q.B; ++b) {
    const __bf16* Hb = static_cast<const __bf16*>(Hs) + (int64_t)b * N * dm;
    const __bf16* Vb = static_cast<const __bf16*>(Vbar) + (int64_t)b * N * dm;
    const __bf16* dOb = static_cast<const __bf16*>(dO) + (int64_t)b * N * dm;
    __bf16* dHb = static_cast<__bf16*>(dHs) + (int64_t)b * N * dm;
    __bf16* dVb = static_cast<__bf16*>(dVbar) + (int64_t)b * N * dm;
    float* R = f32p(oR);
    if (nch == 0) {
      if (!shared) TTT_HIP(zero(dW_down + (int64_t)b * nW, nW));
      continue;
    }
    {
      LaunchTimer lt(K_INP_PREP, st);
      const dim3 tg((unsigned)(dm / 64), (unsigned)(N / 64));
      hipLaunchKernelGGL(transpose_bf16_kernel, tg, dim3(256), 0, st, Hb, bfp(oHt), (int)N, (int)dm);
      hipLaunchKernelGGL(transpose_bf16_kernel, tg, dim3(256), 0, st, Vb, bfp(oVt), (int)N, (int)dm);
      hipLaunchKernelGGL(transpose_bf16_kernel, tg, dim3(256), 0, st, dOb, bfp(odOt), (int)N, (int)dm);
      hipLaunchKernelGGL(transpose_f32_kernel, dim3((unsigned)(dh / 64), (unsigned)(dm / 64)), dim3(256), 0, st,
                         W_down + (int64_t)b * q.wdown_batch_stride, f32p(oWt), bfp(oWtSh), (int)dm, (int)dh);
      TTT_HIP(hipGetLastError());
      TTT_HIP(zero(R, nW));
    }
    // forward sweep: Z_i, Z_i^T, A_i, U_i and the states W_i^T (bf16)
    for (int i = 0; i < nch; ++i) {
      const int64_t zo = (int64_t)i * C * dh;
      Args z{};
      z.A = Hb + (int64_t)i * C * dm;
      z.lda = dm;
      z.B0 = Wg;
      z.B1 = Wu;
      z.ldb = dm;
      z.M = (int)C;
      z.N = (int)dh;
      z.K = (int)dm;
      z.C = bfp(oZ) + zo;
      z.ldc = dh;
      z.Ct = bfp(oZt) + zo;
      z.ldct = C;
      z.Ga = bfp(oGa) + zo;
      z.Gu = bfp(oGu) + zo;
      TTT_HIP(run_gemm<EPI_SWIGLU>(K_INP_Z, z, 1, nullptr, st));
      if (i + 1 < nch)  // W_{i+1}^T = W_i^T + eta Z_i^T Vbar_i
        TTT_HIP(rmw(bfp(oZt) + zo, C, bfp(oVt) + (int64_t)i * C, N, dh, dm, C, f32p(oWt),
                    bfp(oWtSh) + (int64_t)(i + 1) * nW, q.eta));
    }
    // reverse sweep
    for (int i = nch - 1; i >= 0; --i) {
      const int64_t t0 = (int64_t)i * C, zo = (int64_t)i * C * dh;
      const bool later = i + 1 < nch;  // R (the later chunks' gradient) is nonzero
      {
        Args g{};
        g.A = dOb + t0 * dm;
        g.lda = dm;
        g.B0 = bfp(oWtSh) + (int64_t)i * nW;
        g.ldb = dm;
        if (later) {
          g.A2 = Vb + t0 * dm;
          g.B2 = bfp(oRtsh);  // bf16(eta R^T)
          g.K1 = (int)dm;
        }
        g.M = (int)C;
        g.N = (int)dh;
        g.K = (int)(later ? 2 * dm : dm);
        g.Ga = bfp(oGa) + zo;
        g.Gu = bfp(oGu) + zo;
        g.C = bfp(odA);
        g.C2 = bfp(odU);
        g.ldc = dh;
        g.Ct = bfp(odAt) + t0;
        g.Ct2 = bfp(odUt) + t0;
        g.ldct = N;
        TTT_HIP(run_gemm<EPI_SWIGLU_BWD>(K_INP_SWIGLU_BWD, g, 1, nullptr, st));
      }
      if (later) {  // dVbar_i = Z_i bf16(eta R)^T
        TTT_HIP(store(bfp(oZ) + zo, bfp(oRsh), nullptr, nullptr, dh, 0, dh, dm, dVb + t0 * dm, ks_dv));
      } else {
        TTT_HIP(zero(reinterpret_cast<float*>(dVb + t0 * dm), C * dm / 2));  // no later chunk reads its write
      }
      // R += dO_i^T Z_i (shadows eta R and eta R^T for the earlier chunks)
      TTT_HIP(rmw(bfp(odOt) + t0, N, bfp(oZt) + zo, C, dm, dh, C, R, bfp(oRsh), 1.f, q.eta, bfp(oRtsh)));
      // dH_i = dA W_gate + dU W_up
      TTT_HIP(store(bfp(odA), bfp(oWgT), bfp(odU), bfp(oWuT), dh, dh, 2 * dh, dm, dHb + t0 * dm, ks_dh));
    }
    // dW_gate += dA^T H, dW_up += dU^T H over all tokens of the sequence
    TTT_HIP(rmw(bfp(odAt), N, bfp(oHt), N, dh, dm, N, dW_gate, nullptr, 1.f, 1.f, nullptr, K_INP_WGRAD));
    TTT_HIP(rmw(bfp(odUt), N, bfp(oHt), N, dh, dm, N, dW_up, nullptr, 1.f, 1.f, nullptr, K_INP_WGRAD));
    if (shared) {
      hipLaunchKernelGGL(f32_zero_add_kernel, dim3(1024), dim3(256), 0, st, dW_down, static_cast<const float*>(R), nW, 1);
      TTT_HIP(hipGetLastError());
    } else {
      TTT_HIP(hipMemcpyAsync(dW_down + (int64_t)b * nW, R, (size_t)nW * 4, hipMemcpyDeviceToDevice, st));
    }
  }
  return TTT_OK;
}

// ---------------------------------------------------------------------------------------------
// The LM-aligned target on its own ("In-Place Test-Time Training" notes, section 3.2 / Eq. 3):
// Vbar = Conv1D(X0) W_target^T built token-major (ttt_inplace_target_forward), and its gradients
// from dVbar (ttt_inplace_target_backward), so that the target's inputs can be trained through the
// backward of the update. With C = Conv1D(X0) (C[t] = sum_tau taps[tau] * X0[t + tau], zero past
// the end): dC = dVbar W_target (dVbar without a projection), dW_target = sum dVbar^T C,
// dX0[s] = sum_tau taps[tau] * dC[s - tau] (s - tau >= 0), dtaps[tau] = sum_t dC[t] * X0[t + tau].
namespace ttt {

// dX0 tile and per-tile tap partials of one sequence. grid (dm / 64, N / 64), block 256: a 64 x 64
// tile of dX0 from the (64 + k - 1)-row window of dC ending at the tile's last row, and for every
// tap tau the tile's sum over its 64 rows t of dC[t] * X0[t + tau] into part[tile][tau][dm].
__global__ void __launch_bounds__(256) target_conv_bwd_kernel(const __bf16* __restrict__ dC, const __bf16* __restrict__ X0,
                                                             const float* __restrict__ taps, int k, int N, int dm,
                                                             __bf16* __restrict__ dX0, float* __restrict__ part) {
  __shared__ float wd[64 + 15][65];  // dC rows t0 - (k - 1) .. t0 + 63
  __shared__ float wx[64 + 15][65];  // X0 rows t0 .. t0 + 63 + (k - 1)
  __shared__ float tp[16][64];
  __shared__ float red[4][16][64];
  const int c0 = blockIdx.x * 64, t0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int i = tid; i < (64 + k - 1) * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    const int td = t0 - (k - 1) + r, tx = t0 + r;
    wd[r][c] = td >= 0 ? static_cast<float>(dC[(int64_t)td * dm + c0 + c]) : 0.f;
    wx[r][c] = tx < N ? static_cast<float>(X0[(int64_t)tx * dm + c0 + c]) : 0.f;
  }
  for (int i = tid; i < k * 64; i += 256) tp[i / 64][i % 64] = taps[(int64_t)(i / 64) * dm + c0 + i % 64];
  __syncthreads();
  const int c = tid & 63, rq = tid >> 6;  // channel, quarter of the tile's rows
  float acc[16];
#pragma unroll
  for (int tau = 0; tau < 16; ++tau) acc[tau] = 0.f;
  for (int r = rq * 16; r < rq * 16 + 16; ++r) {
    // dX0[t0 + r] = sum_tau taps[tau] dC[t0 + r - tau]; window row of dC[t0 + r - tau] is r + k - 1 - tau
    float s = 0.f;
    for (int tau = 0; tau < k; ++tau) s = fmaf(tp[tau][c], wd[r + k - 1 - tau][c], s);
    dX0[(int64_t)(t0 + r) * dm + c0 + c] = static_cast<__bf16>(s);
    const float d = wd[r + k - 1][c];  // dC[t0 + r]
#pragma unroll
    for (int tau = 0; tau < 16; ++tau)
      if (tau < k) acc[tau] = fmaf(d, wx[r + tau][c], acc[tau]);
  }
#pragma unroll
  for (int tau = 0; tau < 16; ++tau) red[rq][tau][c] = acc[tau];
  __syncthreads();
  for (int i = tid; i < k * 64; i += 256) {
    const int tau = i / 64, cc = i % 64;
    part[((int64_t)blockIdx.y * k + tau) * dm + c0 + cc] = ((red[0][tau][cc] + red[1][tau][cc]) + red[2][tau][cc]) +
                                                           red[3][tau][cc];
  }
}

// dtaps[tau][c] = sum over tiles (in order) of part[tile][tau][c]. grid-stride over k * dm.
__global__ void __launch_bounds__(256) target_taps_sum_kernel(const float* __restrict__ part, int ntiles, int k, int dm,
                                                             float* __restrict__ dtaps) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < k * dm; i += gridDim.x * 256) {
    float s = 0.f;
    for (int t = 0; t < ntiles; ++t) s += part[(int64_t)t * k * dm + i];
    dtaps[i] = s;
  }
}

static ttt_status target_check(const ttt_inplace_params& q) {
  if (q.B < 0 || q.N < 0 || q.d_model <= 0) return TTT_ERR_ARG;
  if (q.dtype != TTT_FP32 && q.dtype != TTT_BF16) return TTT_ERR_ARG;
  if (!q.X0 || !q.conv_taps || q.conv_k < 1 || q.conv_k > 16) return TTT_ERR_ARG;
  if (q.dtype != TTT_BF16) return TTT_ERR_UNSUPPORTED;
  if (q.d_model % 256 || q.N % 128) return TTT_ERR_SHAPE;
  return TTT_OK;
}

}  // namespace ttt

extern "C" ttt_status ttt_inplace_target_forward(const ttt_inplace_params* p, void* Vbar, void* workspace,
                                                 size_t* workspace_bytes, void* stream) {
  using namespace gemm;
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_inplace_params& q = *p;
  const ttt_status chk = target_check(q);
  if (chk != TTT_OK) return chk;
  const int64_t dm = q.d_model, N = q.N;
  if (q.B > 0 && N > 0 && !Vbar) return TTT_ERR_ARG;
  WorkspacePlan plan;
  const size_t oC = plan.add(q.W_target ? (size_t)N * dm * 2 : 0);  // Conv1D(X0) of one sequence
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (q.B == 0 || N == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(gemm_tn_kernel<EPI_STORE>, lds_bytes<EPI_STORE>());
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_STORE>, gemm2::LDS);
    return e;
  }();
  TTT_HIP(lds_ok);
  LaunchTimer lt(K_INP_PREP, st);
  for (int b = 0; b < q.B; ++b) {
    const __bf16* Xb = static_cast<const __bf16*>(q.X0) + (int64_t)b * N * dm;
    __bf16* Vb = static_cast<__bf16*>(Vbar) + (int64_t)b * N * dm;
    __bf16* Cb = q.W_target ? reinterpret_cast<__bf16*>(static_cast<char*>(workspace) + oC) : Vb;
    hipLaunchKernelGGL(target_conv_kernel<false>, dim3((unsigned)(dm / 64), (unsigned)(N / 64)), dim3(256), 0, st, Xb,
                       q.conv_taps, q.conv_k, (int)N, (int)dm, Cb);
    TTT_HIP(hipGetLastError());
    if (q.W_target) {  // Vbar = C W_target^T: A = C [N][in], B = W_target [out][in]
      Args t{};
      t.A = Cb;
      t.lda = dm;
      t.B0 = static_cast<const __bf16*>(q.W_target);
      t.ldb = dm;
      t.M = (int)N;
      t.N = (int)dm;
      t.K = (int)dm;
      t.C = Vb;
      t.ldc = dm;
      TTT_HIP(run_gemm<EPI_STORE>(K_INP_PREP, t, 1, nullptr, st));
    }
  }
  return TTT_OK;
}

extern "C" ttt_status ttt_inplace_target_backward(const ttt_inplace_params* p, const void* dVbar, void* dX0, float* dtaps,
                                                  float* dW_target, void* workspace, size_t* workspace_bytes,
                                                  void* stream) {
  using namespace gemm;
  if (!p || !workspace_bytes) return TTT_ERR_ARG;
  const ttt_inplace_params& q = *p;
  const ttt_status chk = target_check(q);
  if (chk != TTT_OK) return chk;
  const int64_t dm = q.d_model, N = q.N, k = q.conv_k;
  if (q.B > 0 && (!dtaps || (q.W_target != nullptr) != (dW_target != nullptr))) return TTT_ERR_ARG;
  if (q.B > 0 && N > 0 && (!dVbar || !dX0)) return TTT_ERR_ARG;
  const int64_t nt = N / 64;  // token tiles of a sequence
  WorkspacePlan plan;
  const size_t odC = plan.add(q.W_target ? (size_t)N * dm * 2 : 0);   // dC = dVbar W_target
  const size_t oCt = plan.add(q.W_target ? (size_t)dm * N * 2 : 0);   // C^T
  const size_t odVt = plan.add(q.W_target ? (size_t)dm * N * 2 : 0);  // dVbar^T
  const size_t oWtT = plan.add(q.W_target ? (size_t)dm * dm * 2 : 0); // W_target^T
  const size_t oPart = plan.add((size_t)std::max<int64_t>(q.B * nt, 1) * k * dm * 4);
  if (!workspace) {
    *workspace_bytes = plan.total;
    return TTT_OK;
  }
  if (*workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TTT_ERR_WORKSPACE;
  if (q.B == 0) return TTT_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto bfp = [&](size_t o) { return reinterpret_cast<__bf16*>(ws + o); };
  float* part = reinterpret_cast<float*>(ws + oPart);
  static const hipError_t lds_ok = [] {
    hipError_t e = allow_lds(gemm_tn_kernel<EPI_STORE>, lds_bytes<EPI_STORE>());
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_STORE>, gemm2::LDS);
    if (e == hipSuccess) e = allow_lds(gemm2::gemm_big_kernel<EPI_RMW>, gemm2::LDS);
    return e;
  }();
  TTT_HIP(lds_ok);
  LaunchTimer lt(K_INP_PREP, st);
  if (N == 0) {  // no tokens: zero gradients of the taps and the projection
    hipLaunchKernelGGL(f32_zero_add_kernel, dim3(64), dim3(256), 0, st, dtaps, static_cast<const float*>(nullptr), k * dm, 0);
    if (dW_target)
      hipLaunchKernelGGL(f32_zero_add_kernel, dim3(1024), dim3(256), 0, st, dW_target, static_cast<const float*>(nullptr),
                         dm * dm, 0);
    TTT_HIP(hipGetLastError());
    return TTT_OK;
  }
  if (q.W_target) {
    hipLaunchKernelGGL(f32_zero_add_kernel, dim3(1024), dim3(256), 0, st, dW_target, static_cast<const float*>(nullptr),
                       dm * dm, 0);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(dm / 64), (unsigned)(dm / 64)), dim3(256), 0, st,
                       static_cast<const __bf16*>(q.W_target), bfp(oWtT), (int)dm, (int)dm);
    TTT_HIP(hipGetLastError());
  }
  for (int b = 0; b < q.B; ++b) {
    const __bf16* Xb = static_cast<const __bf16*>(q.X0) + (int64_t)b * N * dm;
    const __bf16* dVb = static_cast<const __bf16*>(dVbar) + (int64_t)b * N * dm;
    const __bf16* dC = dVb;
    if (q.W_target) {
      // dW_target += dVbar^T C: A = dVbar^T [out][N], B = C^T [in][N], K = N (one long product)
      hipLaunchKernelGGL(target_conv_kernel<true>, dim3((unsigned)(dm / 64), (unsigned)(N / 64)), dim3(256), 0, st, Xb,
                         q.conv_taps, (int)k, (int)N, (int)dm, bfp(oCt));
      hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(dm / 64), (unsigned)(N / 64)), dim3(256), 0, st, dVb,
                         bfp(odVt), (int)N, (int)dm);
      TTT_HIP(hipGetLastError());
      Args u{};
      u.A = bfp(odVt);
      u.lda = N;
      u.B0 = bfp(oCt);
      u.ldb = N;
      u.M = (int)dm;
      u.N = (int)dm;
      u.K = (int)N;
      u.Wf = dW_target;
      u.Wsh = nullptr;
      u.ldw = dm;
      u.alpha = 1.f;
      TTT_HIP(launch_k(K_INP_PREP, gemm2::gemm_big_kernel<EPI_RMW>, dim3((unsigned)((dm / 256) * (dm / 256))),
                       dim3(gemm2::THREADS), gemm2::LDS, st, u, 1, static_cast<float*>(nullptr)));
      // dC = dVbar W_target: A = dVbar [N][out], B = W_target^T [in][out]
      Args t{};
      t.A = dVb;
      t.lda = dm;
      t.B0 = bfp(oWtT);
      t.ldb = dm;
      t.M = (int)N;
      t.N = (int)dm;
      t.K = (int)dm;
      t.C = bfp(odC);
      t.ldc = dm;
      TTT_HIP(run_gemm<EPI_STORE>(K_INP_PREP, t, 1, nullptr, st));
      dC = bfp(odC);
    }
    hipLaunchKernelGGL(target_conv_bwd_kernel, dim3((unsigned)(dm / 64), (unsigned)nt), dim3(256), 0, st, dC, Xb,
                       q.conv_taps, (int)k, (int)N, (int)dm, static_cast<__bf16*>(dX0) + (int64_t)b * N * dm,
                       part + (int64_t)b * nt * k * dm);
    TTT_HIP(hipGetLastError());
  }
  hipLaunchKernelGGL(target_taps_sum_kernel, dim3((unsigned)((k * dm + 255) / 256)), dim3(256), 0, st, part,
                     (int)(q.B * nt), (int)k, (int)dm, dtaps);
  TTT_HIP(hipGetLastError());
  return TTT_OK;
}
