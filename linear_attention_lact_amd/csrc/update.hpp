// update.hpp -- per-chunk write of the LaCT fast weights (gfx950).
//
// One launch per chunk covers every (pair, matrix) of the call, one workgroup per matrix. For
// each matrix in the update mask ("Test-Time Training Done Right" notes, section 2.2):
//   G = -(sum of the token-segment partial products, in segment order)
//   U = G, or M = momentum * M + G and U = M         (heavy-ball momentum fed to the operator)
//   U = NS5(U) if Muon: X = U / (||U||_F + eps) on the wide orientation X (h x rh), five rounds
//       of A = X X^T, B = b A + c A A, X = a X + B X
//   W = W - U, then each output column renormalised over its inputs to its initial norm
//   fp16/bf16/fp32 operand shadows of the new W for the next chunk's products.
//
// Newton-Schulz is evaluated through the h x h Gram matrix instead of the h x rh iterate. Every
// round multiplies X on the left by P_k = a I + b A_k + c A_k^2 with A_k = X_k X_k^T, so
//   X_5 = Q X_0 with Q = P_4 P_3 P_2 P_1 P_0,  A_{k+1} = P_k A_k P_k
// (P_k is a polynomial in A_k; all of them commute). The result equals the five X rounds up to
// rounding order, while the rounds touch only h x h matrices: X_0 enters twice (A_0 and the
// final Q X_0), streamed from L2 in 64-row chunks, so one workgroup holds a whole matrix and no
// workgroups need to exchange data. Products run in split-bf16 (x = hi + lo, three MFMA products
// per multiply) because the iteration amplifies rounding in weak singular directions by up to
// 3.4445^5; fp32 state, fp32 matrix masters in registers.
#pragma once
#include "common.hpp"

namespace ttt {

constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f;
constexpr int NS_STEPS = 5;

struct LactState {
  float* W;        // [P][3][rh*h]   state rows j, columns c (W0T, W1, W2T)
  float* M;        // [P][3][rh*h]
  float* nu;       // [P][3][NU] renorm targets (W0T/W2T: per row j; W1: per column c)
  void* sh;        // operand shadows [P][4][rh*h] (W0T, W2T, W1, W1T)
  float* part;     // token-segment partial products [S][P][3][rh*h]
  float* U;        // the write before Newton-Schulz [P][3][rh*h] (scratch)
  float* ns;       // global NS5 scratch [P][3][NSZ] (large-h path)
  int P, h, rh, NU;
  int64_t NSZ;
};

struct UpdateArgs {
  LactState s;
  int S;               // token segments
  uint32_t mask;
  int muon, weight_norm;
  float momentum, eps_norm, eps_ns;
};

typedef __bf16 bf16;

__device__ __forceinline__ void split_store(bf16* hi, bf16* lo, float v) {
  const bf16 h = static_cast<bf16>(v);
  *hi = h;
  *lo = static_cast<bf16>(v - static_cast<float>(h));
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// hi / lo bf16 pair of four consecutive values (x = hi + lo to ~2^-16 relative), 8-byte stores
__device__ __forceinline__ void split_store4(bf16* hi, bf16* lo, f32x4 v) {
  bf16x4 h, l;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = static_cast<bf16>(v[q]);
    l[q] = static_cast<bf16>(v[q] - static_cast<float>(h[q]));
  }
  *reinterpret_cast<bf16x4*>(hi) = h;
  *reinterpret_cast<bf16x4*>(lo) = l;
}

template <class T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = Mfma<T>::from_f32(v[q]);
    *reinterpret_cast<t4*>(p) = o;
  }
}

// Split-bf16 product of Q consecutive 32 x 32 output blocks that share their A rows:
//   c[q] += (Ah + Al)[32 x K] (Bh + Bl)[block q]^T, the lo*lo term dropped.
// TA / TB: operand stored K-major (element (k, m) at base[k * ld + m], LDS transpose read);
// otherwise row-major with K contiguous (element (m, k) at base[m * ld + k]).
// B block q starts at Bh + q * 32 (TB) or Bh + q * 32 * ldb. The hi*hi and the cross products
// accumulate in separate registers and are added at the end.
template <int K, int Q, bool TA, bool TB>
__device__ __forceinline__ void mma_split(f32x16 (&c)[Q], const bf16* Ah, const bf16* Al, int lda,
                                          const bf16* Bh, const bf16* Bl, int ldb, int lane) {
  typedef Mfma<bf16> M;
  const int ro = lane & 31, ko = (lane >> 5) * 8;
  f32x16 d[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) zero(d[q]);
#pragma unroll 8
  for (int k = 0; k < K; k += 16) {
    bf16x8 ah, al;
    if constexpr (TA) {
      ah = load_frag_tr<bf16>(Ah, lda, k, lane);
      al = load_frag_tr<bf16>(Al, lda, k, lane);
    } else {
      ah = M::load(Ah + ro * lda + ko + k);
      al = M::load(Al + ro * lda + ko + k);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      bf16x8 bh, bl;
      if constexpr (TB) {
        bh = load_frag_tr<bf16>(Bh + q * 32, ldb, k, lane);
        bl = load_frag_tr<bf16>(Bl + q * 32, ldb, k, lane);
      } else {
        bh = M::load(Bh + (q * 32 + ro) * ldb + ko + k);
        bl = M::load(Bl + (q * 32 + ro) * ldb + ko + k);
      }
      c[q] = M::mma(ah, bh, c[q]);
      d[q] = M::mma(ah, bl, d[q]);
      d[q] = M::mma(al, bh, d[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) c[q] += d[q];
}

// Blocks t = Q*w + q (q < Q) of an NB-block output grid with BPR blocks per row: block t is
// (t / BPR, t % BPR), its A operand the 32-block t / BPR, its B operand the 32-block t % BPR.
// A wave's blocks share their A operand when BPR % Q == 0; otherwise each is formed alone.
template <int K, int Q, int BPR, int NB, bool TA, bool TB>
__device__ __forceinline__ void mma_blocks(f32x16 (&c)[Q], int w, const bf16* Ah, const bf16* Al, int lda,
                                           const bf16* Bh, const bf16* Bl, int ldb, int lane) {
  auto aoff = [&](int b) { return TA ? b * 32 : b * 32 * lda; };
  auto boff = [&](int b) { return TB ? b * 32 : b * 32 * ldb; };
  if constexpr (BPR % Q == 0) {
    const int t0 = Q * w;
    if (t0 < NB)
      mma_split<K, Q, TA, TB>(c, Ah + aoff(t0 / BPR), Al + aoff(t0 / BPR), lda, Bh + boff(t0 % BPR),
                              Bl + boff(t0 % BPR), ldb, lane);
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int t = Q * w + q;
      if (t < NB) {
        f32x16 one[1] = {c[q]};
        mma_split<K, 1, TA, TB>(one, Ah + aoff(t / BPR), Al + aoff(t / BPR), lda, Bh + boff(t % BPR),
                                Bl + boff(t % BPR), ldb, lane);
        c[q] = one[0];
      }
    }
  }
}

// Row stride (16-bit elements) of a chunk read with the LDS transpose read: rows 0..3 of a
// 16-lane group then fall into disjoint 16-bank windows.
constexpr int gram_ld(int h) {
  int l = h + 4;
  while ((l / 2) % 32 != 16) l += 4;
  return l;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int H, int RH>
struct UpdLayout {
  static constexpr int JC = 64;                // state rows per streamed chunk of X^T
  static constexpr int NCH = RH / JC;
  static constexpr int LDA = H + 8;            // h x h matrices: bf16 hi / lo [H][LDA]
  static constexpr int SLOT = 2 * H * LDA * 2;
  static constexpr int LDG = gram_ld(H);       // X^T chunk for the Gram product (transpose reads)
  static constexpr int LDF = H + 8;            // X^T chunk for the final product (row reads)
  static constexpr int CHG = 2 * JC * LDG * 2;
  static constexpr int CHF = 2 * JC * LDF * 2;
  static constexpr int R = cmax(cmax(2 * SLOT, 2 * CHG), SLOT + 2 * CHF);
  static constexpr int HB = H / 32, JBC = JC / 32;
  static constexpr int NF = RH > H ? RH : H;              // renorm factors
  static constexpr int NP = cmax(HB * RH, JBC * H);       // renorm partial sums
  static constexpr int bytes = R + (NP + NF + 32) * 4;
  static constexpr int NBA = HB * HB, QA = (NBA + 7) / 8;   // h x h blocks per wave
  static constexpr int NBF = HB * (JC / 32);                // final-product blocks per chunk
  static_assert(RH % JC == 0 && H % 32 == 0 && NBF <= 8, "shape");
};

template <int H, int RH>
constexpr int update_lds_bytes() { return UpdLayout<H, RH>::bytes; }

// grid: 3 * P workgroups (one per matrix); block 512 threads (8 waves).
// h x h block t = QA*w + q of wave w: rows c = (t / HB)*32 + acc_row, columns
// c' = (t % HB)*32 + acc_col. Every product is stored through its transposed block (the 4
// consecutive accumulator rows of a lane become one 8-byte run), so slot contents are the
// transposes of the masters; each product reads them in the orientation that gives the exact
// (not symmetry-assumed) result wherever a matrix is symmetric only up to rounding: Q's
// dynamic range (up to 3.4445^5 in weak directions) amplifies any such asymmetry.
template <class OpT, int H, int RH>
__device__ __forceinline__ void lact_update_body(const UpdateArgs& u, int mi, unsigned char* smem) {
  typedef UpdLayout<H, RH> L;
  constexpr int JC = L::JC, NCH = L::NCH, LDA = L::LDA, LDG = L::LDG, LDF = L::LDF;
  constexpr int HB = L::HB, NBA = L::NBA, QA = L::QA, NBF = L::NBF;
  constexpr int NE4 = RH * H / 4;              // float4 groups of the matrix
  constexpr int NG = (NE4 + 511) / 512;
  constexpr int CG4 = JC * H / 4 / 512 > 0 ? JC * H / 4 / 512 : 1;   // float4 groups per chunk per thread
  static_assert(JC * H / 4 <= 512 * CG4, "chunk map");
  const LactState& s = u.s;
  bf16* S1h = reinterpret_cast<bf16*>(smem);                 // slot 1 [H][LDA] hi, then lo
  bf16* S1l = S1h + H * LDA;
  bf16* S2h = reinterpret_cast<bf16*>(smem + L::SLOT);       // slot 2
  bf16* S2l = S2h + H * LDA;
  float* npart = reinterpret_cast<float*>(smem + L::R);      // [NP] renorm partial sums
  float* fac = npart + L::NP;                                // [NF] renorm factors
  float* red = fac + L::NF;                                  // [32]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (mi >= 3 * s.P) return;
  const int pair = mi / 3, mat = mi % 3;
  const uint32_t bit = mat == 0 ? 1u : mat == 1 ? 2u : 4u;
  if (!(u.mask & bit)) return;
  const int64_t n = (int64_t)RH * H;
  float* W = s.W + ((int64_t)pair * 3 + mat) * n;
  float* Mm = s.M + ((int64_t)pair * 3 + mat) * n;
  const float* part0 = s.part + ((int64_t)pair * 3 + mat) * n;
  const float* nu = s.nu + ((int64_t)pair * 3 + mat) * s.NU;
  const bool mom = u.momentum != 0.f;
  float* Ud = mom ? Mm : s.U + ((int64_t)pair * 3 + mat) * n;  // U after step 1

  // ---- 1. gradient from the segment partials (in segment order), momentum -------------------
  float ss = 0.f;
  {
    const int64_t seg_stride = (int64_t)s.P * 3 * n;
    constexpr int NB8 = NG < 16 ? NG : 16;
#pragma unroll 1
    for (int b0 = 0; b0 < NG; b0 += NB8) {
      f32x4 g[NB8], mv[NB8];
#pragma unroll
      for (int i = 0; i < NB8; ++i) {
        g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        mv[i] = g[i];
        const int e4 = tid + 512 * (b0 + i);
        if (mom && e4 < NE4) mv[i] = *reinterpret_cast<const f32x4*>(Mm + 4 * e4);
      }
      for (int k = 0; k < u.S; ++k) {
#pragma unroll
        for (int i = 0; i < NB8; ++i) {
          const int e4 = tid + 512 * (b0 + i);
          if (e4 < NE4) g[i] += *reinterpret_cast<const f32x4*>(part0 + k * seg_stride + 4 * e4);
        }
      }
#pragma unroll
      for (int i = 0; i < NB8; ++i) {
        const int e4 = tid + 512 * (b0 + i);
        if (e4 >= NE4) continue;
        f32x4 v = -g[i];
        if (mom) v = u.momentum * mv[i] + v;
        *reinterpret_cast<f32x4*>(Ud + 4 * e4) = v;
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
    }
  }
  float inv = 1.f;
  if (u.muon) inv = 1.f / (sqrtf(block_sum(ss, red)) + u.eps_ns);
  __syncthreads();

  // chunk staging: rows ch*JC .. of U (state rows j, h columns) scaled by inv, as X^T hi / lo.
  // All chunks of the matrix are requested at once (they come from L2: step 1 just wrote them).
  f32x4 cv[NCH][CG4];
  auto chunk_load_all = [&]() {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int i = 0; i < CG4; ++i) {
        const int e4 = tid + 512 * i;
        cv[ch][i] = e4 < JC * H / 4 ? *reinterpret_cast<const f32x4*>(Ud + (int64_t)ch * JC * H + 4 * e4)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  auto chunk_store = [&](int ch, bf16* bh, bf16* bl, int ld) {
#pragma unroll
    for (int c4 = 0; c4 < NCH; ++c4) {
      if (c4 != ch) continue;
#pragma unroll
      for (int i = 0; i < CG4; ++i) {
        const int e4 = tid + 512 * i;
        if (e4 < JC * H / 4) {
          const int row = (4 * e4) / H, c = (4 * e4) % H;
          split_store4(bh + row * ld + c, bl + row * ld + c, cv[c4][i] * inv);
        }
      }
    }
  };
  auto put_sym = [&](const f32x16 (&v)[QA], bf16* dh, bf16* dl) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int t = QA * w + q;
      if (t < NBA) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c = (t / HB) * 32 + 8 * g4 + 4 * (lane >> 5), c2 = (t % HB) * 32 + (lane & 31);
          split_store4(dh + c2 * LDA + c, dl + c2 * LDA + c,
                       f32x4{v[q][4 * g4], v[q][4 * g4 + 1], v[q][4 * g4 + 2], v[q][4 * g4 + 3]});
        }
      }
    }
  };
  // the same blocks stored in their own orientation (element [c][c'] at row c): 2-byte stores,
  // used once for Q, which the final product reads by rows
  auto put_direct = [&](const f32x16 (&v)[QA], bf16* dh, bf16* dl) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int t = QA * w + q;
      if (t < NBA) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = (t / HB) * 32 + acc_row(r, lane), c2 = (t % HB) * 32 + acc_col(lane);
          const bf16 hi = static_cast<bf16>(v[q][r]);
          dh[c * LDA + c2] = hi;
          dl[c * LDA + c2] = static_cast<bf16>(v[q][r] - static_cast<float>(hi));
        }
      }
    }
  };
  auto zero_q = [&](f32x16 (&v)[QA]) {
#pragma unroll
    for (int q = 0; q < QA; ++q) zero(v[q]);
  };

  // ---- 2. Newton-Schulz-5 through the Gram matrix ----------------------------------------------
  if (u.muon) {
    f32x16 am[QA], pm[QA], qm[QA], t[QA];
    // (a) A_0 = X_0 X_0^T, X_0^T streamed in chunks of JC state rows (double-buffered)
    zero_q(am);
    {
      auto gb = [&](int i) { return reinterpret_cast<bf16*>(smem + (i & 1) * L::CHG); };
      chunk_load_all();
      chunk_store(0, gb(0), gb(0) + JC * LDG, LDG);
      __syncthreads();
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        if (ch + 1 < NCH) {
          bf16* nb = gb(ch + 1);
          chunk_store(ch + 1, nb, nb + JC * LDG, LDG);
        }
        bf16* cb = gb(ch);
        mma_blocks<JC, QA, HB, NBA, true, true>(am, w, cb, cb + JC * LDG, LDG, cb, cb + JC * LDG, LDG, lane);
        __syncthreads();
      }
    }
    put_sym(am, S1h, S1l);
    __syncthreads();
    // (b) five rounds on h x h matrices: slot 1 holds A_k (then P_k A_k, then Q_k), slot 2 P_k
#pragma unroll 1
    for (int k = 0; k < NS_STEPS; ++k) {
      zero_q(t);
      mma_blocks<H, QA, HB, NBA, false, false>(t, w, S1h, S1l, LDA, S1h, S1l, LDA, lane);  // A_k^2
#pragma unroll
      for (int q = 0; q < QA; ++q) {
        const int tb = QA * w + q;
        const bool diag = (tb / HB) == (tb % HB);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float id = (diag && acc_row(r, lane) == acc_col(lane)) ? NS_A : 0.f;
          pm[q][r] = id + NS_B * am[q][r] + NS_C * t[q][r];
        }
      }
      put_sym(pm, S2h, S2l);
      __syncthreads();
      if (k + 1 < NS_STEPS) {
        // C = A^T P^T (slot 1 rows, slot 2 read K-major), stored transposed: slot 1 <- P A in
        // its own orientation (P A is symmetric only up to rounding, which the rounds amplify)
        zero_q(t);
        mma_blocks<H, QA, HB, NBA, false, true>(t, w, S1h, S1l, LDA, S2h, S2l, LDA, lane);
        __syncthreads();
        put_sym(t, S1h, S1l);
        __syncthreads();
        zero_q(am);
        mma_blocks<H, QA, HB, NBA, false, false>(am, w, S1h, S1l, LDA, S2h, S2l, LDA, lane);  // (P A) P
        __syncthreads();
      }
      if (k == 0) {
#pragma unroll
        for (int q = 0; q < QA; ++q) qm[q] = pm[q];
      } else {
        put_sym(qm, S1h, S1l);
        __syncthreads();
        zero_q(qm);
        mma_blocks<H, QA, HB, NBA, false, false>(qm, w, S2h, S2l, LDA, S1h, S1l, LDA, lane);  // P Q
        __syncthreads();
      }
      if (k + 1 < NS_STEPS) {
        put_sym(am, S1h, S1l);
        __syncthreads();
      }
    }
    put_direct(qm, S1h, S1l);  // Q in slot 1, row-major, for the final product
    __syncthreads();
  }

  // ---- 3. W - U per chunk, U = (Q X_0)^T with Muon: block C[c][j] = sum_m Q[c][m] X_0^T[j][m] ---
  // wave w < NBF owns block (c-block w / (JC/32), j-block w % (JC/32)) of every chunk and keeps
  // the new state of those blocks in registers through the renorm and the writes
  constexpr int JBC = L::JBC;
  const bool fact = w < NBF;
  const int fcb = (w < NBF ? w : 0) / JBC, fjb = (w < NBF ? w : 0) % JBC;
  auto fcoord = [&](int ch, int g4, int& j, int& c) {
    c = fcb * 32 + 8 * g4 + 4 * (lane >> 5);
    j = ch * JC + fjb * 32 + (lane & 31);
  };
  f32x16 wn[NCH];
  if (fact) {  // all of this wave's W entries in flight at once
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        int j, c;
        fcoord(ch, g4, j, c);
        const f32x4 wv = *reinterpret_cast<const f32x4*>(W + (int64_t)j * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) wn[ch][4 * g4 + i] = wv[i];
      }
  }
  {
    auto fb = [&](int i) { return reinterpret_cast<bf16*>(smem + L::SLOT + (i & 1) * L::CHF); };
    if (u.muon) {
      chunk_load_all();
      chunk_store(0, fb(0), fb(0) + JC * LDF, LDF);
      __syncthreads();
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      f32x16 cx[1];
      zero(cx[0]);
      if (u.muon) {
        if (ch + 1 < NCH) {
          bf16* nb = fb(ch + 1);
          chunk_store(ch + 1, nb, nb + JC * LDF, LDF);
        }
        bf16* cb = fb(ch);
        mma_blocks<H, 1, JBC, NBF, false, false>(cx, w, S1h, S1l, LDA, cb, cb + JC * LDF, LDF, lane);
      }
      if (fact) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          int j, c;
          fcoord(ch, g4, j, c);
          f32x4 uv;
          if (u.muon)
            uv = f32x4{cx[0][4 * g4], cx[0][4 * g4 + 1], cx[0][4 * g4 + 2], cx[0][4 * g4 + 3]};
          else
            uv = *reinterpret_cast<const f32x4*>(Ud + (int64_t)j * H + c);
#pragma unroll
          for (int i = 0; i < 4; ++i) wn[ch][4 * g4 + i] -= uv[i];
        }
      }
      if (u.muon) __syncthreads();
    }
  }

  // ---- 4. renorm over the input axis (partial sums of squares from the register blocks) --------
  if (u.weight_norm) {
    if (mat == 1) {  // W1 [rh][h]: column c over all rh rows; lanes of a half hold 32 rows j
      if (fact) {
        float cs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float a = 0.f;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) a += wn[ch][r] * wn[ch][r];
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) a += __shfl_xor(a, off, 64);
          cs[r] = a;
        }
        if ((lane & 31) == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) npart[fjb * H + fcb * 32 + acc_row(r, lane)] = cs[r];
        }
      }
      __syncthreads();
      for (int c = tid; c < H; c += 512) {
        float tot = 0.f;
        for (int jb = 0; jb < JBC; ++jb) tot += npart[jb * H + c];
        fac[c] = nu[c] / (sqrtf(tot) + u.eps_norm);
      }
    } else {  // W0T / W2T: state row j over its h inputs; a lane holds 16 of a block's 32 columns
      if (fact) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          float a = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) a += wn[ch][r] * wn[ch][r];
          a += __shfl_xor(a, 32, 64);
          if (lane < 32) npart[fcb * RH + ch * JC + fjb * 32 + lane] = a;
        }
      }
      __syncthreads();
      for (int j = tid; j < RH; j += 512) {
        float tot = 0.f;
        for (int cb = 0; cb < HB; ++cb) tot += npart[cb * RH + j];
        fac[j] = nu[j] / (sqrtf(tot) + u.eps_norm);
      }
    }
    __syncthreads();
  }

  // ---- 5. state and operand shadows from the register blocks ----------------------------------
  if (fact) {
    OpT* sh = reinterpret_cast<OpT*>(s.sh) + (int64_t)pair * 4 * n;
    OpT* dst = sh + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        int j, c;
        fcoord(ch, g4, j, c);
        f32x4 v = f32x4{wn[ch][4 * g4], wn[ch][4 * g4 + 1], wn[ch][4 * g4 + 2], wn[ch][4 * g4 + 3]};
        if (u.weight_norm) {
          if (mat == 1)
            v *= *reinterpret_cast<const f32x4*>(fac + c);
          else
            v *= fac[j];
        }
        *reinterpret_cast<f32x4*>(W + (int64_t)j * H + c) = v;
        store4(dst + (int64_t)j * H + c, v);
        if (mat == 1) {  // W1^T shadow [h][rh]: 32 lanes write 32 consecutive j of a row c
#pragma unroll
          for (int i = 0; i < 4; ++i) sh[3 * n + (int64_t)(c + i) * RH + j] = Mfma<OpT>::from_f32(v[i]);
        }
      }
  }
}

// workgroup mi handles matrix mi % 3 of pair mi / 3
template <class OpT, int H, int RH>
__global__ void __launch_bounds__(512) lact_update_kernel(UpdateArgs u) {
  extern __shared__ __align__(16) unsigned char smem[];
  lact_update_body<OpT, H, RH>(u, blockIdx.x, smem);
}

}  // namespace ttt
