// update.hpp -- batched per-matrix write of the LaCT fast weights (gfx950).
//
// One launch per chunk covers every (pair, matrix) of the call. For each matrix in the
// update mask ("Test-Time Training Done Right" notes, section 2.2):
//   G = -(sum of the token-segment partial products, in segment order)
//   U = G, or M = momentum * M + G and U = M         (heavy-ball momentum fed to the operator)
//   U = NS5(U) if Muon: X = U / (||U||_F + eps), five rounds of
//       A = X X^T, B = b A + c A A, X = a X + B X, on the wide orientation X (h x rh)
//   W = W - U, then each output column renormalised over its inputs to its initial norm
//   fp16/bf16/fp32 operand shadows of the new W for the next chunk's products.
// Newton-Schulz runs in split-bf16 (x = hi + lo, three MFMA products per multiply) because the
// iteration amplifies rounding in weak singular directions by up to 3.4445^5; fp32 state.
//
// Work split: the wide X is split by columns into G parts (G = 2 for rh = 256), one
// workgroup each, both on the same XCD. Each workgroup keeps its X columns and the full h x h
// Gram / polynomial matrix in LDS (fp32) and forms bf16 hi/lo fragments on the fly. Per round
// the partial Gram matrices are exchanged through L2 (xcd_sync.hpp); A^2 is formed redundantly
// by both workgroups so that one exchange per round suffices.
#pragma once
#include "common.hpp"
#include "xcd_sync.hpp"

namespace ttt {

constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f;
constexpr int NS_STEPS = 5;

struct LactState {
  float* W;        // [P][3][rh*h]   state rows j, columns c (W0T, W1, W2T)
  float* M;        // [P][3][rh*h]
  float* nu;       // [P][3][NU] renorm targets (W0T/W2T: per row j; W1: per column c)
  void* sh;        // operand shadows [P][4][rh*h] (W0T, W2T, W1, W1T)
  float* part;     // token-segment partial products [S][P][3][rh*h]
  float* ns;       // global NS5 scratch [P][3][NSZ] (large-h path)
  float* xbuf;     // exchange buffers [P*3][2 parity][2 parts][h*h]
  unsigned* sync;  // [P*3][SYNC_LINE] barrier counters, then error word at sync[P*3*SYNC_LINE]
  int P, h, rh, NU;
  int64_t NSZ;
};

struct UpdateArgs {
  LactState s;
  int S;               // token segments
  uint32_t mask;
  int muon, weight_norm;
  float momentum, eps_norm, eps_ns;
  int chunk;           // chunk index (barrier targets continue across launches)
};

typedef __bf16 bf16;

__device__ __forceinline__ void split_store(bf16* hi, bf16* lo, float v) {
  const bf16 h = static_cast<bf16>(v);
  *hi = h;
  *lo = static_cast<bf16>(v - static_cast<float>(h));
}

// Split-bf16 products for a 32 x 64 output block (two 32 x 32 tiles sharing the A rows):
//   c_t += (Ah + Al)[32 x K] * (Bh + Bl)^T, dropping the lo*lo term.
// A rows are K-contiguous (lda). B is either n-major (rows n, K-contiguous; TR = false) or
// K-major (rows k, n-contiguous; TR = true, read with the LDS transpose read). `two` = false
// computes only the first tile.
template <int K, bool TR>
__device__ __forceinline__ void mma_split_2t(f32x16& c0, f32x16& c1, const bf16* Ah, const bf16* Al, int lda,
                                             const bf16* Bh, const bf16* Bl, int ldb, bool two, int lane) {
  typedef Mfma<bf16> M;
  const int ao = (lane & 31) * lda + (lane >> 5) * 8;
  const int bo = (lane & 31) * ldb + (lane >> 5) * 8;
#pragma unroll 1
  for (int k = 0; k < K; k += 16) {
    const bf16x8 ah = M::load(Ah + ao + k), al = M::load(Al + ao + k);
    bf16x8 b0h, b0l, b1h, b1l;
    if constexpr (TR) {
      b0h = load_frag_tr<bf16>(Bh, ldb, k, lane);
      b0l = load_frag_tr<bf16>(Bl, ldb, k, lane);
    } else {
      b0h = M::load(Bh + bo + k);
      b0l = M::load(Bl + bo + k);
    }
    c0 = M::mma(ah, b0h, c0);
    c0 = M::mma(ah, b0l, c0);
    c0 = M::mma(al, b0h, c0);
    if (two) {
      if constexpr (TR) {
        b1h = load_frag_tr<bf16>(Bh + 32, ldb, k, lane);
        b1l = load_frag_tr<bf16>(Bl + 32, ldb, k, lane);
      } else {
        b1h = M::load(Bh + 32 * ldb + bo + k);
        b1l = M::load(Bl + 32 * ldb + bo + k);
      }
      c1 = M::mma(ah, b1h, c1);
      c1 = M::mma(ah, b1l, c1);
      c1 = M::mma(al, b1h, c1);
    }
  }
}

template <int H, int RH, int G>
struct UpdLayout {
  static constexpr int RHG = RH / G;          // X columns (state rows) per workgroup
  static constexpr int LDX = RHG + 8;         // bf16 row stride of X hi / lo  [H][LDX]
  static constexpr int LDA = H + 8;           // bf16 row stride of A hi / lo  [H][LDA]
  static constexpr int LDW = RHG + 4;         // fp32 row stride of the new W  [H][LDW]
  static constexpr int XB = 2 * H * LDX * 2;  // bytes of X hi + lo
  static constexpr int AB = 2 * H * LDA * 2;
  static constexpr int WB = H * LDW * 4;
  static constexpr int RB = AB > WB ? AB : WB; // A hi/lo and the new W share one region
  static constexpr int bytes = XB + RB + (2 * H + 32) * 4;
};

template <int H, int RH, int G>
constexpr int update_lds_bytes() { return UpdLayout<H, RH, G>::bytes; }

// grid: G * 8 * ceil(M / 8) workgroups for M = 3 * P matrices (G == 2: the parts of a matrix
// are workgroups w and w + 8, i.e. on one XCD); block 512 threads (8 waves).
template <class OpT, int H, int RH, int G>
__global__ void __launch_bounds__(512) lact_update_kernel(UpdateArgs u) {
  static_assert(G == 1 || G == 2, "parts");
  typedef UpdLayout<H, RH, G> L;
  constexpr int RHG = L::RHG, LDX = L::LDX, LDA = L::LDA, LDW = L::LDW;
  constexpr int HB = H / 32, CB = RHG / 32;
  constexpr int NWV = 8;
  const LactState& s = u.s;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Xh = reinterpret_cast<bf16*>(smem);                 // [H][LDX]  X columns of this part
  bf16* Xl = Xh + H * LDX;
  bf16* Ah = reinterpret_cast<bf16*>(smem + L::XB);         // [H][LDA]  Gram / polynomial matrix
  bf16* Al = Ah + H * LDA;
  float* Wn = reinterpret_cast<float*>(smem + L::XB);       // [H][LDW]  new W (after Newton-Schulz)
  float* cn = reinterpret_cast<float*>(smem + L::XB + L::RB);  // [2H]
  float* red = cn + 2 * H;                                  // [32]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wg = blockIdx.x;
  const int part = G == 2 ? ((wg >> 3) & 1) : 0;
  const int mi = G == 2 ? ((wg & 7) + 8 * (wg >> 4)) : wg;
  const int M = 3 * s.P;
  if (mi >= M) return;
  const int pair = mi / 3, mat = mi % 3;
  const uint32_t bit = mat == 0 ? 1u : mat == 1 ? 2u : 4u;
  if (!(u.mask & bit)) return;
  unsigned* err = s.sync + (size_t)M * SYNC_LINE;
  unsigned* cnt = s.sync + (size_t)mi * SYNC_LINE;
  if (G == 2 && tid == 0 && hw_xcc_id() != (unsigned)(wg & 7))
    __hip_atomic_fetch_add(err, 1u << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nb = G == 2 ? (u.muon ? 1 + NS_STEPS : 0) + (mat == 1 && u.weight_norm ? 1 : 0) : 0;
  int bi = u.chunk * nb;  // barriers completed by this matrix before this launch
  float* xb = s.xbuf + (size_t)mi * 4 * H * H;
  auto xslot = [&](int parity, int p) { return xb + ((size_t)parity * 2 + p) * H * H; };

  const int64_t n = (int64_t)RH * H;
  const int j0 = part * RHG;
  float* W = s.W + ((int64_t)pair * 3 + mat) * n;
  float* Mm = s.M + ((int64_t)pair * 3 + mat) * n;
  const float* nu = s.nu + ((int64_t)pair * 3 + mat) * s.NU;

  // ---- 1. gradient from the segment partials (in segment order), momentum -------------------
  // U is staged transposed in the (still unused) fp32 W region: Wn[c][jl] = U[j0 + jl][c]
  {
    const int64_t seg_stride = (int64_t)s.P * 3 * n;
    const float* pp = s.part + ((int64_t)pair * 3 + mat) * n;
    float ss = 0.f;
    // float4 groups of 4 consecutive c; all segment loads of a group issued together
#pragma unroll 2
    for (int e4 = tid; e4 < RHG * H / 4; e4 += 512) {
      const int jl = (4 * e4) / H, c = (4 * e4) % H;
      const int64_t idx = (int64_t)(j0 + jl) * H + c;
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < u.S; ++k) g += *reinterpret_cast<const f32x4*>(pp + k * seg_stride + idx);
      g = -g;
      f32x4 v = g;
      if (u.momentum != 0.f) {
        v = u.momentum * *reinterpret_cast<const f32x4*>(Mm + idx) + g;
        *reinterpret_cast<f32x4*>(Mm + idx) = v;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Wn[(c + q) * LDW + jl] = v[q];
        ss += v[q] * v[q];
      }
    }
    float inv = 1.f;
    if (u.muon) {
      float tot = block_sum(ss, red);
      if constexpr (G == 2) {
        float* mine = xslot(bi & 1, part);
        if (tid == 0) mine[0] = tot;
        xcd_barrier(cnt, G * (++bi), err);
        const float* m0 = xslot((bi - 1) & 1, 0);
        const float* m1 = xslot((bi - 1) & 1, 1);
        tot = xcd_load(m0) + xcd_load(m1);
      }
      inv = 1.f / (sqrtf(tot) + u.eps_ns);
    }
    __syncthreads();
    // X[c][jl] = U[j0 + jl][c] * inv, as hi / lo
    for (int e = tid; e < H * RHG; e += 512) {
      const int c = e / RHG, jl = e % RHG;
      split_store(Xh + c * LDX + jl, Xl + c * LDX + jl, Wn[c * LDW + jl] * inv);
    }
    __syncthreads();
  }

  // ---- 2. Newton-Schulz-5 ------------------------------------------------------------------
  if (u.muon) {
    constexpr int PB_A = HB * ((HB + 1) / 2);   // 32 x 64 units of an H x H product
    constexpr int PB_X = HB * ((CB + 1) / 2);   // 32 x 64 units of the H x RHG product
    for (int it = 0; it < NS_STEPS; ++it) {
      // (a) Gram partial over this part's columns (one 32 x 64 unit per wave at most)
      static_assert(PB_A <= NWV, "Gram units per wave");
      {
        const int t = w < PB_A ? w : 0;
        const bool active = w < PB_A;
        const int ib = t / ((HB + 1) / 2), kb = 2 * (t % ((HB + 1) / 2));
        const bool two = active && kb + 1 < HB;
        f32x16 c0, c1;
        zero(c0);
        zero(c1);
        if (active)
          mma_split_2t<RHG, false>(c0, c1, Xh + ib * 32 * LDX, Xl + ib * 32 * LDX, LDX, Xh + kb * 32 * LDX,
                                   Xl + kb * 32 * LDX, LDX, two, lane);
        if constexpr (G == 1) {
          if (active) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = ib * 32 + acc_row(r, lane), k = kb * 32 + acc_col(lane);
              split_store(Ah + i * LDA + k, Al + i * LDA + k, c0[r]);
              if (two) split_store(Ah + i * LDA + k + 32, Al + i * LDA + k + 32, c1[r]);
            }
          }
        } else {
          // own partial to L2; after the barrier add the partner's at the same positions
          // (IEEE addition commutes, so both parts form bitwise the same A)
          float* mine = xslot(bi & 1, part);
          if (active) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = ib * 32 + acc_row(r, lane), k = kb * 32 + acc_col(lane);
              mine[i * H + k] = c0[r];
              if (two) mine[i * H + k + 32] = c1[r];
            }
          }
          xcd_barrier(cnt, G * (++bi), err);
          const float* other = xslot((bi - 1) & 1, part ^ 1);
          if (active) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = ib * 32 + acc_row(r, lane), k = kb * 32 + acc_col(lane);
              c0[r] += xcd_load(other + i * H + k);
              if (two) c1[r] += xcd_load(other + i * H + k + 32);
            }
          }
          if (active)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = ib * 32 + acc_row(r, lane), k = kb * 32 + acc_col(lane);
            split_store(Ah + i * LDA + k, Al + i * LDA + k, c0[r]);
            if (two) split_store(Ah + i * LDA + k + 32, Al + i * LDA + k + 32, c1[r]);
          }
        }
      }
      __syncthreads();
      // (b) B = b A + c A A   (A symmetric: its rows serve as the n-major B operand)
      {
        constexpr int NQ = (PB_A + NWV - 1) / NWV;
        f32x16 q0[NQ], q1[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int t = w + q * NWV;
          zero(q0[q]);
          zero(q1[q]);
          if (t < PB_A) {
            const int ib = t / ((HB + 1) / 2), kb = 2 * (t % ((HB + 1) / 2));
            mma_split_2t<H, false>(q0[q], q1[q], Ah + ib * 32 * LDA, Al + ib * 32 * LDA, LDA, Ah + kb * 32 * LDA,
                                   Al + kb * 32 * LDA, LDA, kb + 1 < HB, lane);
          }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int t = w + q * NWV;
          if (t < PB_A) {
            const int ib = t / ((HB + 1) / 2), kb = 2 * (t % ((HB + 1) / 2));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = ib * 32 + acc_row(r, lane), k = kb * 32 + acc_col(lane);
              const int o = i * LDA + k;
              split_store(Ah + o, Al + o, NS_B * (static_cast<float>(Ah[o]) + static_cast<float>(Al[o])) + NS_C * q0[q][r]);
              if (kb + 1 < HB)
                split_store(Ah + o + 32, Al + o + 32,
                            NS_B * (static_cast<float>(Ah[o + 32]) + static_cast<float>(Al[o + 32])) + NS_C * q1[q][r]);
            }
          }
        }
        __syncthreads();
      }
      // (c) X = a X + B X over this part's columns (X read K-major with the transpose read)
      {
        constexpr int NQ = (PB_X + NWV - 1) / NWV;
        f32x16 q0[NQ], q1[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int t = w + q * NWV;
          zero(q0[q]);
          zero(q1[q]);
          if (t < PB_X) {
            const int ib = t / ((CB + 1) / 2), jb = 2 * (t % ((CB + 1) / 2));
            mma_split_2t<H, true>(q0[q], q1[q], Ah + ib * 32 * LDA, Al + ib * 32 * LDA, LDA, Xh + jb * 32,
                                  Xl + jb * 32, LDX, jb + 1 < CB, lane);
          }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int t = w + q * NWV;
          if (t < PB_X) {
            const int ib = t / ((CB + 1) / 2), jb = 2 * (t % ((CB + 1) / 2));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int o = (ib * 32 + acc_row(r, lane)) * LDX + jb * 32 + acc_col(lane);
              split_store(Xh + o, Xl + o, NS_A * (static_cast<float>(Xh[o]) + static_cast<float>(Xl[o])) + q0[q][r]);
              if (jb + 1 < CB)
                split_store(Xh + o + 32, Xl + o + 32,
                            NS_A * (static_cast<float>(Xh[o + 32]) + static_cast<float>(Xl[o + 32])) + q1[q][r]);
            }
          }
        }
        __syncthreads();
      }
    }
  }

  // ---- 3. W = W - U, kept as Wn[c][jl] (fp32); renorm over the input axis -----------------------
  // U = hi + lo (the split pair carries U to ~2^-16 relative, also without Muon)
#pragma unroll 4
  for (int e4 = tid; e4 < RHG * H / 4; e4 += 512) {
    const int jl = (4 * e4) / H, c = (4 * e4) % H;
    const f32x4 wv = *reinterpret_cast<const f32x4*>(W + (int64_t)(j0 + jl) * H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = (c + q) * LDX + jl;
      Wn[(c + q) * LDW + jl] = wv[q] - (static_cast<float>(Xh[o]) + static_cast<float>(Xl[o]));
    }
  }
  __syncthreads();
  if (u.weight_norm) {
    if (mat == 1) {  // W1 [rh][h]: column c over all rh rows (both parts)
      for (int c = w; c < H; c += NWV) {
        float acc = 0.f;
        for (int jl = lane; jl < RHG; jl += 64) acc += Wn[c * LDW + jl] * Wn[c * LDW + jl];
        acc = wave_sum(acc);
        if (lane == 0) cn[c] = acc;
      }
      if constexpr (G == 2) {
        __syncthreads();
        float* mine = xslot(bi & 1, part);
        for (int c = tid; c < H; c += 512) mine[c] = cn[c];
        xcd_barrier(cnt, G * (++bi), err);
        const float* m0 = xslot((bi - 1) & 1, 0);
        const float* m1 = xslot((bi - 1) & 1, 1);
        for (int c = tid; c < H; c += 512) cn[c] = xcd_load(m0 + c) + xcd_load(m1 + c);
      }
      __syncthreads();
      for (int c = tid; c < H; c += 512) cn[H + c] = nu[c] / (sqrtf(cn[c]) + u.eps_norm);
      __syncthreads();
      for (int e = tid; e < H * RHG; e += 512) Wn[(e / RHG) * LDW + e % RHG] *= cn[H + e / RHG];
    } else {  // W0T / W2T: row j over its h inputs (column jl of Wn)
      for (int jl = tid; jl < RHG; jl += 512) {
        float acc = 0.f;
        for (int c = 0; c < H; ++c) acc += Wn[c * LDW + jl] * Wn[c * LDW + jl];
        const float f = nu[j0 + jl] / (sqrtf(acc) + u.eps_norm);
        for (int c = 0; c < H; ++c) Wn[c * LDW + jl] *= f;
      }
    }
    __syncthreads();
  }
  // ---- 4. state and operand shadows -----------------------------------------------------------
  OpT* sh = reinterpret_cast<OpT*>(s.sh) + (int64_t)pair * 4 * n;
  OpT* dst = sh + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n;
  for (int e = tid; e < RHG * H; e += 512) {
    const int jl = e / H, c = e % H;
    const float v = Wn[c * LDW + jl];
    const int64_t idx = (int64_t)(j0 + jl) * H + c;
    W[idx] = v;
    dst[idx] = Mfma<OpT>::from_f32(v);
  }
  if (mat == 1) {
    for (int e = tid; e < RHG * H; e += 512) {
      const int c = e / RHG, jl = e % RHG;
      sh[3 * n + (int64_t)c * RH + j0 + jl] = Mfma<OpT>::from_f32(Wn[c * LDW + jl]);
    }
  }
}

}  // namespace ttt
