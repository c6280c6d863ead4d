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
#include "fastweight.hpp"

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
  float* esc;      // power-of-two step-size scales of the gradient segments [chunk][P][S]
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

// hi / lo bf16 pair of four consecutive values (x = hi + lo to ~2^-16 relative), 8-byte stores.
// hi is the round-to-nearest bf16 pair; its fp32 values come from the bit pattern (a shift and a
// mask) rather than a second conversion.
__device__ __forceinline__ void split4(f32x4 v, bf16x4& h, bf16x4& l) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const bf16x2 hp = __builtin_convertvector(f32x2{v[2 * p], v[2 * p + 1]}, bf16x2);
    const unsigned hb = __builtin_bit_cast(unsigned, hp);
    const float h0 = __builtin_bit_cast(float, hb << 16), h1 = __builtin_bit_cast(float, hb & 0xffff0000u);
    const bf16x2 lp = __builtin_convertvector(f32x2{v[2 * p] - h0, v[2 * p + 1] - h1}, bf16x2);
    h[2 * p] = hp[0];
    h[2 * p + 1] = hp[1];
    l[2 * p] = lp[0];
    l[2 * p + 1] = lp[1];
  }
}
__device__ __forceinline__ void split_store4(bf16* hi, bf16* lo, f32x4 v) {
  bf16x4 h, l;
  split4(v, h, l);
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

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Row stride (bf16 elements) of the h x h slots: the smallest 16-byte multiple >= h + 8 whose
// 4-byte word count is 12 mod 32. Measured at h = 128 (304-byte rows): the row reads run as with
// 272-byte rows and the transpose reads of the P A product lose their bank conflicts (1.5 us per
// product instead of 2.2); 288-byte rows slow every product down.
constexpr int slot_ld(int h) {
  int l = h + 8;
  while ((l / 2) % 32 != 12) l += 8;
  return l;
}

template <int H, int RH>
struct UpdLayout {
  static constexpr int LDA = slot_ld(H);       // h x h matrices: bf16 hi / lo [H][LDA]
  static constexpr int SLOT = 2 * H * LDA * 2;
  typedef TileLayout<__bf16, H> GL;            // X_0^T (rows j, h columns) for the Gram product
  static constexpr int GSZ = RH * GL::LD;      // elements of its hi (and of its lo) array
  static constexpr int R = cmax(2 * SLOT, 2 * GSZ * 2);
  static constexpr int HB = H / 32, NJ = RH / 32;
  static constexpr int NJW = (NJ + 7) / 8;     // state-row blocks per wave in the final product
  static constexpr int bytes = R + (8 * H + 32) * 4;      // + column-norm partials [8][H], [32]
  static constexpr int NBA = HB * HB, QA = (NBA + 7) / 8;   // h x h blocks per wave
  static_assert(H % 32 == 0 && RH % 32 == 0 && bytes <= 160 * 1024, "shape");
};

template <int H, int RH>
constexpr int update_lds_bytes() { return UpdLayout<H, RH>::bytes; }

// Gram product A_0 = X_0 X_0^T for the Q consecutive 32 x 32 blocks of one block row starting at
// block t0 = (t0 / HB, t0 % HB): K runs over all RH state rows of X_0^T (transpose reads of the
// swizzled rows; both operands take the same permuted K order), split-bf16 with the cross terms
// in separate registers.
template <class GL, int RH, int Q, int HB>
__device__ __forceinline__ void gram_row(f32x16 (&c)[Q], int t0, const bf16* Gh, const bf16* Gl, int lane) {
  typedef Mfma<bf16> M;
  const int ca = 32 * (t0 / HB), cb0 = 32 * (t0 % HB);
  f32x16 d[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) zero(d[q]);
#pragma unroll 2
  for (int hr = 0; hr < RH / 32; ++hr) {
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const bf16x8 ah = tile_kfrag_tr<GL>(Gh, 32 * hr, ca, q2, lane);
      const bf16x8 al = tile_kfrag_tr<GL>(Gl, 32 * hr, ca, q2, lane);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const bf16x8 bh = tile_kfrag_tr<GL>(Gh, 32 * hr, cb0 + 32 * q, q2, lane);
        const bf16x8 bl = tile_kfrag_tr<GL>(Gl, 32 * hr, cb0 + 32 * q, q2, lane);
        c[q] = M::mma(ah, bh, c[q]);
        d[q] = M::mma(ah, bl, d[q]);
        d[q] = M::mma(al, bh, d[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) c[q] += d[q];
}

// wave w's blocks t = Q*w + q of the h x h Gram matrix (one block row when HB % Q == 0)
template <class GL, int RH, int Q, int HB, int NBA>
__device__ __forceinline__ void gram_blocks(f32x16 (&c)[Q], int w, const bf16* Gh, const bf16* Gl, int lane) {
  if constexpr (HB % Q == 0) {
    if (Q * w < NBA) gram_row<GL, RH, Q, HB>(c, Q * w, Gh, Gl, lane);
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int t = Q * w + q;
      if (t < NBA) {
        f32x16 one[1] = {c[q]};
        gram_row<GL, RH, 1, HB>(one, t, Gh, Gl, lane);
        c[q] = one[0];
      }
    }
  }
}

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
  typedef typename L::GL GL;
  constexpr int LDA = L::LDA, HB = L::HB, NBA = L::NBA, QA = L::QA, NJ = L::NJ, NJW = L::NJW;
  constexpr int NE4 = RH * H / 4;              // float4 groups of the matrix
  constexpr int NG = (NE4 + 511) / 512;
  constexpr int NB8 = NG < 16 ? NG : 16;
  constexpr bool KEEP = NG <= NB8;             // step 1 holds the whole matrix in registers
  const LactState& s = u.s;
  bf16* S1h = reinterpret_cast<bf16*>(smem);                 // slot 1 [H][LDA] hi, then lo
  bf16* S1l = S1h + H * LDA;
  bf16* S2h = reinterpret_cast<bf16*>(smem + L::SLOT);       // slot 2
  bf16* S2l = S2h + H * LDA;
  float* npart = reinterpret_cast<float*>(smem + L::R);      // [8][H] column-norm partials
  float* red = npart + 8 * H;                                // [32]

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
  f32x4 keep[KEEP ? NG : 1];
  {
    const int64_t seg_stride = (int64_t)s.P * 3 * n;
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
        f32x4 v = -g[i];
        if (mom) v = u.momentum * mv[i] + v;
        if constexpr (KEEP) keep[i] = v;
        if (e4 >= NE4) continue;
        *reinterpret_cast<f32x4*>(Ud + 4 * e4) = v;
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
    }
  }
  // The norm needs LDS only: its barriers leave the U stores in flight (they drain during the
  // staging below, whose barrier waits for them; every later read of U follows that barrier).
  float inv = 1.f;
  if (u.muon) {
    ss = wave_sum(ss);
    lds_barrier();
    if (lane == 0) red[w] = ss;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) tot += red[i];
    inv = 1.f / (sqrtf(tot) + u.eps_ns);
  } else {
    __syncthreads();
  }

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
    // (a) X_0^T = U^T / (||U||_F + eps) as split-bf16 rows j in LDS, then A_0 = X_0 X_0^T in one
    //     pass over all RH rows
    {
      bf16* Gh = reinterpret_cast<bf16*>(smem);
      bf16* Gl = Gh + L::GSZ;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int e4 = tid + 512 * i;
        if (NE4 % 512 == 0 || e4 < NE4) {
          f32x4 v;
          if constexpr (KEEP)
            v = keep[i];
          else
            v = *reinterpret_cast<const f32x4*>(Ud + 4 * e4);  // this thread's own step-1 writes
          const int j = (4 * e4) / H, c = (4 * e4) % H;
          split_store4(Gh + GL::at(j, c), Gl + GL::at(j, c), v * inv);
        }
      }
      __syncthreads();
      zero_q(am);
      gram_blocks<GL, RH, QA, HB, NBA>(am, w, Gh, Gl, lane);
      __syncthreads();
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

  // ---- 3-5. new state: wave w takes the state rows of blocks jb = w, w + 8, ... and keeps every
  // h column of them in registers through W - U, the renorm and the writes. With Muon the write
  // is U = (Q X_0)^T, each lane loading its X_0^T row j straight from the step-1 output as
  // split-bf16 operand fragments (k = m = 16 s + 8 (lane / 32) + e), Q read by rows from slot 1.
  // Block orientation per matrix, so that the renorm axis lies along the lane's own registers:
  //   W0T / W2T (norm of row j over its h inputs): blocks C[c][j], a lane holds one j;
  //   W1 (norm of column c over all rh rows): blocks C[j][c], a lane holds one c.
  auto finish = [&](auto ROWS_J) {
    constexpr bool RJ = decltype(ROWS_J)::value;  // accumulator rows are state rows j (W1)
    constexpr int KS = H / 16;
    f32x16 wn[NJW][HB];
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int jb = w + 8 * x;
      if (jb < NJ) {
        const int jl = 32 * jb + (lane & 31);
        if (u.muon) {
          bf16x8 uh[KS], ul[KS];
#pragma unroll
          for (int st = 0; st < KS; ++st) {
            const float* src = Ud + (int64_t)jl * H + 16 * st + 8 * (lane >> 5);
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(src) * inv;
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4) * inv;
            bf16x4 h0, l0, h1, l1;
            split4(v0, h0, l0);
            split4(v1, h1, l1);
            uh[st] = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
            ul[st] = bf16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
          }
          f32x16 dd[HB];
#pragma unroll
          for (int cb = 0; cb < HB; ++cb) {
            zero(wn[x][cb]);
            zero(dd[cb]);
          }
#pragma unroll
          for (int st = 0; st < KS; ++st) {
#pragma unroll
            for (int cb = 0; cb < HB; ++cb) {
              const int qo = (32 * cb + (lane & 31)) * LDA + 16 * st + 8 * (lane >> 5);
              const bf16x8 qh = Mfma<bf16>::load(S1h + qo), ql = Mfma<bf16>::load(S1l + qo);
              if constexpr (RJ) {
                wn[x][cb] = Mfma<bf16>::mma(uh[st], qh, wn[x][cb]);
                dd[cb] = Mfma<bf16>::mma(uh[st], ql, dd[cb]);
                dd[cb] = Mfma<bf16>::mma(ul[st], qh, dd[cb]);
              } else {
                wn[x][cb] = Mfma<bf16>::mma(qh, uh[st], wn[x][cb]);
                dd[cb] = Mfma<bf16>::mma(qh, ul[st], dd[cb]);
                dd[cb] = Mfma<bf16>::mma(ql, uh[st], dd[cb]);
              }
            }
          }
#pragma unroll
          for (int cb = 0; cb < HB; ++cb) wn[x][cb] += dd[cb];
        } else {
#pragma unroll
          for (int cb = 0; cb < HB; ++cb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int ro = 8 * g4 + 4 * (lane >> 5);
              if constexpr (RJ) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  wn[x][cb][4 * g4 + i] = Ud[(int64_t)(32 * jb + ro + i) * H + 32 * cb + (lane & 31)];
              } else {
                const f32x4 v = *reinterpret_cast<const f32x4*>(Ud + (int64_t)jl * H + 32 * cb + ro);
#pragma unroll
                for (int i = 0; i < 4; ++i) wn[x][cb][4 * g4 + i] = v[i];
              }
            }
        }
        // W - U
#pragma unroll
        for (int cb = 0; cb < HB; ++cb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int ro = 8 * g4 + 4 * (lane >> 5);
            if constexpr (RJ) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                wn[x][cb][4 * g4 + i] = W[(int64_t)(32 * jb + ro + i) * H + 32 * cb + (lane & 31)] - wn[x][cb][4 * g4 + i];
            } else {
              const f32x4 v = *reinterpret_cast<const f32x4*>(W + (int64_t)jl * H + 32 * cb + ro);
#pragma unroll
              for (int i = 0; i < 4; ++i) wn[x][cb][4 * g4 + i] = v[i] - wn[x][cb][4 * g4 + i];
            }
          }
      }
    }

    // renorm over the input axis to the initial norms
    float fr[NJW];      // W0T / W2T: factor of this lane's row j in block x
    float fc[HB];       // W1: factor of this lane's column c in block cb
#pragma unroll
    for (int x = 0; x < NJW; ++x) fr[x] = 1.f;
#pragma unroll
    for (int cb = 0; cb < HB; ++cb) fc[cb] = 1.f;
    if (u.weight_norm) {
      if constexpr (RJ) {
#pragma unroll
        for (int cb = 0; cb < HB; ++cb) {
          float a = 0.f;
#pragma unroll
          for (int x = 0; x < NJW; ++x)
            if (w + 8 * x < NJ) {
#pragma unroll
              for (int r = 0; r < 16; ++r) a += wn[x][cb][r] * wn[x][cb][r];
            }
          a += __shfl_xor(a, 32, 64);
          if (lane < 32) npart[w * H + 32 * cb + lane] = a;
        }
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < HB; ++cb) {
          const int c = 32 * cb + (lane & 31);
          float tot = 0.f;
#pragma unroll
          for (int v = 0; v < 8; ++v) tot += npart[v * H + c];
          fc[cb] = nu[c] / (sqrtf(tot) + u.eps_norm);
        }
      } else {
#pragma unroll
        for (int x = 0; x < NJW; ++x) {
          const int jb = w + 8 * x;
          if (jb < NJ) {
            float a = 0.f;
#pragma unroll
            for (int cb = 0; cb < HB; ++cb)
#pragma unroll
              for (int r = 0; r < 16; ++r) a += wn[x][cb][r] * wn[x][cb][r];
            a += __shfl_xor(a, 32, 64);
            fr[x] = nu[32 * jb + (lane & 31)] / (sqrtf(a) + u.eps_norm);
          }
        }
      }
    }

    // state and operand shadows
    OpT* sh = reinterpret_cast<OpT*>(s.sh) + (int64_t)pair * 4 * n;
    OpT* dst = sh + (mat == 0 ? 0 : mat == 2 ? 1 : 2) * n;
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int jb = w + 8 * x;
      if (jb < NJ) {
        const int jl = 32 * jb + (lane & 31);
#pragma unroll
        for (int cb = 0; cb < HB; ++cb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int ro = 8 * g4 + 4 * (lane >> 5);
            f32x4 v = f32x4{wn[x][cb][4 * g4], wn[x][cb][4 * g4 + 1], wn[x][cb][4 * g4 + 2], wn[x][cb][4 * g4 + 3]};
            if constexpr (RJ) {  // rows j0 .. j0 + 3 of column c
              v *= fc[cb];
              const int j0 = 32 * jb + ro, c = 32 * cb + (lane & 31);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                W[(int64_t)(j0 + i) * H + c] = v[i];
                dst[(int64_t)(j0 + i) * H + c] = Mfma<OpT>::from_f32(v[i]);
              }
              store4(sh + 3 * n + (int64_t)c * RH + j0, v);  // W1^T shadow [h][rh]
            } else {             // columns c0 .. c0 + 3 of row j
              v *= fr[x];
              const int c0 = 32 * cb + ro;
              *reinterpret_cast<f32x4*>(W + (int64_t)jl * H + c0) = v;
              store4(dst + (int64_t)jl * H + c0, v);
            }
          }
      }
    }
  };
  if (mat == 1)
    finish(std::true_type{});
  else
    finish(std::false_type{});
}

// workgroup mi handles matrix mi % 3 of pair mi / 3
template <class OpT, int H, int RH>
__global__ void __launch_bounds__(512) lact_update_kernel(UpdateArgs u) {
  extern __shared__ __align__(16) unsigned char smem[];
  lact_update_body<OpT, H, RH>(u, blockIdx.x, smem);
}

}  // namespace ttt
