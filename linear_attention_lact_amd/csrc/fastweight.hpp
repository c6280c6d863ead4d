// fastweight.hpp -- gfx950 kernels for the SwiGLU fast weight f(x) = (silu(x W0) * (x W2)) W1
// (row-vector form; bias free). Shared by the LaCT layer and its linear-attention form.
//
// Stored layouts (per (sequence, head) pair, operand type OpT):
//   W0T, W2T [rh][H]  -- W0, W2 transposed: row j holds the input weights of hidden unit j
//   W1       [rh][H]  -- row j holds the output weights of hidden unit j
//   W1T      [H][rh]
// Token tensors are [pair][N][H] in the I/O type, step sizes [pair][N] float.
//
// grad_kernel: for a token range of one chunk and a block of 64 hidden units, computes the
// positive partial sums
//     P0 = K^T X0,  P1 = (eta*H)^T V,  P2 = K^T X2   (stored transposed as [j][c])
// with A = K W0, Bm = K W2, D = eta * (V W1^T), H = silu(A)*Bm, X0 = D*Bm*silu'(A),
// X2 = D*silu(A). The loss -sum eta <f(k), v> has gradients G0 = -P0, G1 = -P1, G2 = -P2
// ("Test-Time Training Done Right" notes, section 2.2; the chain rule through the SwiGLU).
// In linear-attention mode only P1 = phi(K)^T diag(eta) V is formed (the chunk aggregate of
// the scan form; KV-binding summary page, "Prerequisites -> Linear attention").
// Every hidden unit j only touches column j of W0/W2 and row j of W1, so hidden-unit blocks
// are independent; token ranges are summed afterwards in a fixed order.
//
// apply_kernel: O = (silu(Q W0) * (Q W2)) W1 for a tile of 64 query tokens, streaming the
// hidden dimension in blocks of 64.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace ttt {

constexpr int RB = 64;   // hidden units per block
constexpr int TT = 64;   // tokens per tile
constexpr int NWAVE = 4; // waves per workgroup (256 threads)

template <class T> struct Pad { static constexpr int v = 16 / sizeof(T); };  // 16-byte row pad

struct GradArgs {
  const void* K;          // [pair][N][H] I/O type
  const void* V;
  const float* eta;       // [pair][N]
  int64_t tok_pair_stride;   // elements between pairs in K/V (= N*H)
  int64_t eta_pair_stride;   // (= N)
  int t_base;             // first token of the region (chunk start)
  int seg_len;            // tokens per grid.y segment
  int t_limit;            // one past the last token of the region
  const void* W0T;        // [rh][H] operand type, per pair
  const void* W2T;
  const void* W1;
  int64_t w_pair_stride;  // elements between pairs of the shadows
  int rh;
  float* out;             // partial sums, fp32
  int64_t out_y_stride;   // between grid.y segments
  int64_t out_pair_stride;
  int64_t out_mat_stride; // between P0 / P1 / P2 (= rh*H)
  const float* eta_scale; // [pair][segment] power-of-two step-size scales of the region
                          // (grad_ws_kernel; the other kernels derive them themselves)
  int64_t eta_mat_stride; // E3 kernels: between the step-size rows of W0, W1, W2 (eta [pair][3][N])
};
// E3 (eta per matrix): the gradient of W_X uses its own step-size row eta_X: eta_1 scales H in
// P1 = (eta_1 H)^T V, eta_0 and eta_2 scale D in X0 and X2.

// K-major fragment: element (k, n) at base[k * ld + n]; lane l receives n = l & 31 and the
// k values of its K step (16-bit: LDS transpose read; fp32: one strided element).
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_kmajor(const T* base, int ld, int k0, int lane) {
  if constexpr (sizeof(T) == 2) {
    return load_frag_tr<T>(base, ld, k0, lane);
  } else {
    return base[(k0 + (lane >> 5)) * ld + (lane & 31)];
  }
}

// Staging of a 64-token tile of K and V: each thread moves NCH 16-byte chunks per tensor from
// global memory (rows beyond the segment are zero) through registers into row-major LDS
// [t][c], converting to the operand type on the way.
template <class IoT, class OpT, int H, int NTHR = 256>
struct TileStage {
  static constexpr int VE = Io<IoT>::VEC;                 // elements per 16-byte chunk
  static constexpr int NCH = TT * H / VE / NTHR;          // chunks per thread per tensor (NTHR threads)
  static_assert(TT * H % (VE * NTHR) == 0, "staging map");
  u32x4 k[NCH], v[NCH];
  __device__ __forceinline__ void load(const IoT* Kp, const IoT* Vp, int t0, int t_end, int tid) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = tid + NTHR * q;
      const int row = ch / (H / VE), col = (ch % (H / VE)) * VE;
      if (t0 + row < t_end) {
        k[q] = *reinterpret_cast<const u32x4*>(Kp + (int64_t)(t0 + row) * H + col);
        v[q] = *reinterpret_cast<const u32x4*>(Vp + (int64_t)(t0 + row) * H + col);
      } else {
        k[q] = u32x4{0u, 0u, 0u, 0u};
        v[q] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ static void put(const u32x4& raw, OpT* dst) {
    if constexpr (sizeof(IoT) == 2 && std::is_same<OpT, _Float16>::value) {  // 8 bf16 -> 8 fp16
      *reinterpret_cast<f16x8*>(dst) = bf16x8_to_f16x8(raw);
    } else if constexpr (sizeof(IoT) == 2) {
      const u16x8 b = __builtin_bit_cast(u16x8, raw);
      typename Mfma<OpT>::frag f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = Mfma<OpT>::from_f32(bf16_to_f32(b[e]));
      *reinterpret_cast<typename Mfma<OpT>::frag*>(dst) = f;
    } else {                           // 4 fp32
      *reinterpret_cast<u32x4*>(dst) = raw;
    }
  }
  template <class TL>
  __device__ __forceinline__ void store_at(OpT* Ks, OpT* Vs, int tid) const {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = tid + NTHR * q;
      const int row = ch / (H / VE), col = (ch % (H / VE)) * VE;
      put(k[q], Ks + TL::at(row, col));
      put(v[q], Vs + TL::at(row, col));
    }
  }
  __device__ __forceinline__ void store(OpT* Ks, OpT* Vs, int ld, int tid) const {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = tid + NTHR * q;
      const int row = ch / (H / VE), col = (ch % (H / VE)) * VE;
      put(k[q], Ks + row * ld + col);
      put(v[q], Vs + row * ld + col);
    }
  }
};

// Token-tile layout of the register-direct kernels. With 16-bit operands and h = 128 the rows
// carry no padding and the 16-byte chunk c of row r sits at position c ^ (4 (r % 4) + (r / 4) % 2):
// the MFMA row reads (8 consecutive rows of one chunk), the transpose reads (4 rows x 32
// columns) and the 16-byte staging writes then each touch distinct LDS banks. Other shapes pad
// the rows by 16 bytes.
template <class OpT, int H>
struct TileLayout {
  static constexpr bool SWZ = sizeof(OpT) == 2 && H == 128;
  static constexpr int LD = SWZ ? H : H + Pad<OpT>::v;
  __device__ __forceinline__ static int at(int r, int c) {
    if constexpr (SWZ)
      return r * LD + (((c >> 3) ^ (4 * (r & 3) + ((r >> 2) & 1))) << 3) + (c & 7);
    else
      return r * LD + c;
  }
};

// Transpose-read operand (see acc_kfrag_tr) from a tile in TileLayout: rows row0.. (tokens),
// columns col0.. .
template <class TL, class T>
__device__ __forceinline__ typename Mfma<T>::frag tile_kfrag_tr(const T* tile, int row0, int col0, int q, int lane) {
  if constexpr (!TL::SWZ) {
    return acc_kfrag_tr<T>(tile + row0 * TL::LD + col0, TL::LD, q, lane);
  } else {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    const int g = lane >> 4, s = lane & 15;
    const int row = row0 + 16 * q + 4 * (g >> 1) + (s >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
    v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4*)((__attribute__((address_space(3))) T*)(tile + TL::at(row, col))));
    v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4*)((__attribute__((address_space(3))) T*)(tile + TL::at(row + 8, col))));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(typename Mfma<T>::frag, v);
  }
}

// LDS bytes of grad_kernel<OpT, H, LINATTN>.
template <class OpT, int H, bool LINATTN, bool E3 = false>
constexpr int grad_lds_bytes() {
  constexpr int P = Pad<OpT>::v;
  constexpr int nW = LINATTN ? 2 : 3;
  constexpr int nMid = LINATTN ? 1 : 3;
  return (nW * RB * (H + P) + 2 * TT * (H + P) + nMid * RB * (TT + P)) * (int)sizeof(OpT) + (E3 ? 3 : 1) * TT * 4 +
         16 * 4;
}

// grid: x = hidden block (rh/64), y = token segment, z = pair. block: 64 NWV threads (NWV waves).
// Per 64-token tile: K and V are staged row-major in LDS by all threads (the next tile is
// prefetched into registers meanwhile); wave (th, jh) < 4 forms A^T, Bm^T, D^T for hidden rows
// jh*32.. and tokens th*32.. (operands: fast-weight rows and token rows, both K-contiguous), the
// SwiGLU / silu' epilogue writes eta*H, X0, X2 as [j][t] tiles, and the token contractions, split
// over all NWV waves, read K and V K-major through the LDS transpose read. With eight waves (two
// per SIMD) each wave holds half the contraction accumulators of the four-wave form, and the
// register file takes both.
template <class IoT, class OpT, int H, bool LINATTN, bool SCALE_MID, bool E3 = false, int NWV = NWAVE>
__global__ void __launch_bounds__(64 * NWV) grad_kernel(GradArgs a) {
  static_assert(!(E3 && LINATTN), "one step size per token in linear-attention mode");
  constexpr int NE = E3 ? 3 : 1;  // step-size rows
  typedef Mfma<OpT> M;
  constexpr int P = Pad<OpT>::v;
  constexpr int LDW = H + P;        // W block / token tile row stride
  constexpr int LDT = TT + P;       // mid row stride
  constexpr int nW = LINATTN ? 2 : 3;
  constexpr int nMid = LINATTN ? 1 : 3;
  constexpr int NMAT = LINATTN ? 1 : 3;
  constexpr int CB = H / 32;                       // 32-wide column blocks of H
  constexpr int NQ = NMAT * 2 * CB;                // gradient C tiles per workgroup
  constexpr int NT = (NQ + NWV - 1) / NWV;         // per wave
  constexpr int KS = H / M::KSTEP;                 // K steps over H
  constexpr int NTH = 64 * NWV;                    // threads; waves 4.. only join the contractions

  extern __shared__ __align__(16) unsigned char smem[];
  OpT* Wb = reinterpret_cast<OpT*>(smem);                    // [nW][RB][LDW]
  OpT* Ks = Wb + nW * RB * LDW;                              // [TT][LDW]
  OpT* Vs = Ks + TT * LDW;                                   // [TT][LDW]
  OpT* Mid = Vs + TT * LDW;                                  // [nMid][RB][LDT]
  float* eta_s = reinterpret_cast<float*>(Mid + nMid * RB * LDT);  // [NE][TT]
  float* red = eta_s + NE * TT;                              // [16]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int jb = blockIdx.x, seg = blockIdx.y, pair = blockIdx.z;
  const int t_begin = a.t_base + seg * a.seg_len;
  const int t_end = min(t_begin + a.seg_len, a.t_limit);

  const IoT* Kp = reinterpret_cast<const IoT*>(a.K) + pair * a.tok_pair_stride;
  const IoT* Vp = reinterpret_cast<const IoT*>(a.V) + pair * a.tok_pair_stride;
  const float* ep = a.eta + pair * a.eta_pair_stride;

  TileStage<IoT, OpT, H, NTH> stage;
  stage.load(Kp, Vp, t_begin, t_end, tid);

  // --- stage this hidden block of the fast weights ---------------------------------------
  {
    const OpT* src[3] = {reinterpret_cast<const OpT*>(a.W0T), reinterpret_cast<const OpT*>(a.W2T),
                         reinterpret_cast<const OpT*>(a.W1)};
    constexpr int VPR = H * (int)sizeof(OpT) / 16;  // 16-byte vectors per row
    for (int m = 0; m < nW; ++m) {
      const OpT* s = src[m] + pair * a.w_pair_stride + (int64_t)jb * RB * H;
      for (int i = tid; i < RB * VPR; i += NTH) {
        const int row = i / VPR, v = i % VPR;
        *reinterpret_cast<u32x4*>(Wb + (m * RB + row) * LDW + v * (16 / sizeof(OpT))) =
            *reinterpret_cast<const u32x4*>(s + row * H + v * (16 / sizeof(OpT)));
      }
    }
  }

  // --- power-of-two scale keeping eta-scaled intermediates in the operand range ---------
  float scale = 1.f;
  if constexpr (SCALE_MID) {
    float mx = 0.f;
    for (int e = 0; e < NE; ++e)
      for (int t = t_begin + tid; t < t_end; t += NTH) mx = fmaxf(mx, ep[e * a.eta_mat_stride + t]);
    mx = block_max(mx, red);
    if (mx > 0.f) scale = exp2f(-floorf(log2f(mx)));
  }

  f32x16 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) zero(acc[i]);

  const int th = w >> 1, jh = w & 1;  // forward role: token half, hidden half
  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    __syncthreads();  // previous tile's LDS reads are done
    stage.store(Ks, Vs, LDW, tid);
    if (tid < NE * TT) {
      const int e = tid / TT, t = tid % TT;
      eta_s[tid] = (t0 + t < t_end) ? ep[e * a.eta_mat_stride + t0 + t] * scale : 0.f;
    }
    __syncthreads();
    if (t0 + TT < t_end) stage.load(Kp, Vp, t0 + TT, t_end, tid);  // in flight during the MFMAs

    // forward products for (hidden rows jh*32.., tokens th*32..): A^T, Bm^T, D^T
    if (w < 4) {
      f32x16 fa, fb, fd;
      zero(fa);
      zero(fb);
      zero(fd);
      const OpT* w0 = Wb + (0 * RB + jh * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
      const OpT* w2 = Wb + (1 * RB + jh * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
      const OpT* w1 = Wb + (2 * RB + jh * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
      const OpT* kr = Ks + (th * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
      const OpT* vr = Vs + (th * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const auto kf = M::load(kr + s * M::KSTEP);
        fa = M::mma(M::load(w0 + s * M::KSTEP), kf, fa);
        fb = M::mma(M::load(w2 + s * M::KSTEP), kf, fb);
        if constexpr (!LINATTN) fd = M::mma(M::load(w1 + s * M::KSTEP), M::load(vr + s * M::KSTEP), fd);
      }
      // epilogue: element (j, t) with j = jh*32 + acc_row, t = th*32 + lane&31
      const int tl = th * 32 + (lane & 31);
      const float e = eta_s[(E3 ? TT : 0) + tl];                 // eta (eta_1 with E3)
      const float e0 = E3 ? eta_s[tl] : e, e2 = E3 ? eta_s[2 * TT + tl] : e;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jh * 32 + acc_row(r, lane);
        const float A = fa[r], Bm = fb[r];
        const float sg = sigmoidf_(A);
        const float sil = A * sg;
        Mid[(0 * RB + j) * LDT + tl] = M::from_f32(e * sil * Bm);  // eta * H
        if constexpr (!LINATTN) {
          Mid[(1 * RB + j) * LDT + tl] = M::from_f32(e0 * fd[r] * Bm * (sg * (1.f + A * (1.f - sg))));  // X0
          Mid[(2 * RB + j) * LDT + tl] = M::from_f32(e2 * fd[r] * sil);                                 // X2
        }
      }
    }
    __syncthreads();  // Mid visible

    // token contractions: P1 += (eta H)^T V, P0 += X0^T K, P2 += X2^T K (rows j, cols c)
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int q = w + NWV * i;
      if (q < NQ) {
        const int mat = q / (2 * CB), jhq = (q / CB) % 2, cb = q % CB;
        const OpT* am = Mid + (mat * RB + jhq * 32 + (lane & 31)) * LDT + (lane >> 5) * M::KSUB;
        const OpT* bt = (mat == 0 ? Vs : Ks) + cb * 32;
#pragma unroll
        for (int k = 0; k < TT; k += M::KSTEP)
          acc[i] = M::mma(M::load(am + k), load_frag_kmajor<OpT>(bt, LDW, k, lane), acc[i]);
      }
    }
  }

  // --- write partial sums: rows j, cols c; out matrices ordered (P0, P1, P2) ---------------
  const float inv = 1.f / scale;
  float* ob = a.out + seg * a.out_y_stride + pair * a.out_pair_stride;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int q = w + NWV * i;
    if (q < NQ) {
      const int mat = q / (2 * CB), jhq = (q / CB) % 2, cb = q % CB;
      const int omat = LINATTN ? 0 : (mat == 0 ? 1 : (mat == 1 ? 0 : 2));
      float* o = ob + omat * a.out_mat_stride + ((int64_t)jb * RB + jhq * 32) * H + cb * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[acc_row(r, lane) * H + acc_col(lane)] = acc[i][r] * inv;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Register-direct variant for h <= 128 (same arguments and outputs as grad_kernel).
// Wave w = jh + 2 th forms the forward products of hidden rows jh*32.. (of the workgroup's 64)
// and token half th of every 64-token tile. Its slices of W0^T, W2^T, W1 stay in registers as
// MFMA B fragments for the whole segment. The forward products are formed as C[t][j] (K and V
// rows as the A operand, from the row-major LDS tile), so the epilogue values eta*H, X0, X2
// serve directly as A fragments of the token contractions (acc_to_afrag). For the contractions
// the wave takes column half th of the h outputs over all 64 tokens: its own A fragments come
// from registers, its partner's (same jh, other token half) through a small LDS exchange, and
// the K / V fragments from the LDS tile through the permuted transpose read (acc_kfrag_tr).
// Every output element is thus summed by one wave in a fixed order.
// Software pipeline: K, V and eta tiles are double-buffered in LDS and the tile after next is
// prefetched into registers; the forward MFMAs of tile i+1 are interleaved with the (VALU)
// epilogue of tile i, so matrix cores and vector ALU overlap within the single wave per SIMD
// that the register budget allows.
// Block mapping: the hidden blocks of one (pair, segment) are workgroups w, w+8, ..., i.e. on
// one XCD, so its K / V tiles are fetched from HBM once per XCD.
// grid: x = rh/64 * 8 * ceil(P * nseg / 8); block 256.
template <class OpT, int H, bool LINATTN, bool E3 = false>
constexpr int grad_rd_lds_bytes() {
  constexpr int P = Pad<OpT>::v;
  constexpr int NMAT = LINATTN ? 1 : 3;
  constexpr int QS = 32 / Mfma<OpT>::KSTEP;
  constexpr int FRAG = (int)sizeof(typename Mfma<OpT>::frag);
  (void)P;
  return 4 * TT * TileLayout<OpT, H>::LD * (int)sizeof(OpT) + (2 * (E3 ? 3 : 1) * TT + 16) * 4 +
         NWAVE * NMAT * QS * 64 * FRAG;
}

// sigmoid through the hardware exp2 and reciprocal (about 1 ulp each; the results feed 16-bit
// MFMA operands). Saturates to 0 / 1 for large |a|.
__device__ __forceinline__ float sigmoid_fast(float a) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}

template <class IoT, class OpT, int H, bool LINATTN, bool SCALE_MID, bool E3 = false>
__global__ void __launch_bounds__(256) grad_rd_kernel(GradArgs a, int nseg, int npairs) {
  static_assert(H <= 128, "register budget");
  static_assert(!(E3 && LINATTN), "one step size per token in linear-attention mode");
  constexpr int NE = E3 ? 3 : 1;  // step-size rows
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  constexpr int P = Pad<OpT>::v;
  typedef TileLayout<OpT, H> TL;
  constexpr int LDK = TL::LD;
  constexpr int TILE = TT * LDK;            // elements of one staged tensor tile
  constexpr int CB = H / 32;
  constexpr int CH = (CB + 1) / 2;          // output column blocks per wave
  constexpr int KS = H / M::KSTEP;          // forward K steps over h
  constexpr int QS = 32 / M::KSTEP;         // contraction K steps over a 32-token half
  constexpr int NMAT = LINATTN ? 1 : 3;
  constexpr int NWM = LINATTN ? 2 : 3;

  extern __shared__ __align__(16) unsigned char smem[];
  OpT* tiles = reinterpret_cast<OpT*>(smem);                  // [2 buffers][K, V][TT][LDK]
  float* eta_s = reinterpret_cast<float*>(tiles + 4 * TILE);  // [2 buffers][NE][TT]
  float* red = eta_s + 2 * NE * TT;                           // [16]
  frag* xch = reinterpret_cast<frag*>(red + 16);              // [NWAVE][NMAT][QS][64]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int njb = a.rh / RB;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int jb = slot % njb;
  const int group = xcd + 8 * (slot / njb);
  if (group >= npairs * nseg) return;
  const int pair = group / nseg, seg = group % nseg;
  const int t_begin = a.t_base + seg * a.seg_len;
  const int t_end = min(t_begin + a.seg_len, a.t_limit);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + TT - 1) / TT : 0;
  const int jh = w & 1, th = w >> 1;
  const int cb0 = th * CH;                  // first output column block of this wave

  const IoT* Kp = reinterpret_cast<const IoT*>(a.K) + pair * a.tok_pair_stride;
  const IoT* Vp = reinterpret_cast<const IoT*>(a.V) + pair * a.tok_pair_stride;
  const float* ep = a.eta + pair * a.eta_pair_stride;

  TileStage<IoT, OpT, H> stage;
  float ev = 0.f;
  auto fetch = [&](int i) {
    const int t0 = t_begin + i * TT;
    stage.load(Kp, Vp, t0, t_end, tid);
    if (tid < NE * TT) {
      const int e = tid / TT, t = tid % TT;
      ev = (t0 + t < t_end) ? ep[e * a.eta_mat_stride + t0 + t] : 0.f;
    }
  };
  if (ntiles > 0) fetch(0);

  // fast-weight slices as B fragments: lane (n = j, k = c) of rows jb*64 + jh*32 + (lane & 31)
  frag wf[NWM][KS];
  {
    const OpT* src[3] = {reinterpret_cast<const OpT*>(a.W0T), reinterpret_cast<const OpT*>(a.W2T),
                         reinterpret_cast<const OpT*>(a.W1)};
#pragma unroll
    for (int m = 0; m < NWM; ++m) {
      const OpT* row = src[m] + pair * a.w_pair_stride + (int64_t)(jb * RB + jh * 32 + (lane & 31)) * H +
                       (lane >> 5) * M::KSUB;
#pragma unroll
      for (int s = 0; s < KS; ++s) wf[m][s] = M::load(row + s * M::KSTEP);
    }
  }

  float scale = 1.f;
  if constexpr (SCALE_MID) {
    float mx = 0.f;
    for (int e = 0; e < NE; ++e)
      for (int t = t_begin + tid; t < t_end; t += 256) mx = fmaxf(mx, ep[e * a.eta_mat_stride + t]);
    mx = block_max(mx, red);
    if (mx > 0.f) scale = exp2f(-floorf(log2f(mx)));
  }
  auto put = [&](int i) {
    OpT* b = tiles + (i & 1) * 2 * TILE;
    stage.template store_at<TL>(b, b + TILE, tid);
    if (tid < NE * TT) eta_s[(i & 1) * NE * TT + tid] = ev * scale;
  };

  f32x16 acc[NMAT][CH];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CH; ++c) zero(acc[m][c]);

  // forward of the tile in buffer `b` (tokens th*32.., hidden jh*32..) into F, with the epilogue
  // of the previous tile's Fp (eta from ebuf) interleaved when EPI is set:
  // Fp[0] <- eta*H, Fp[1] <- X0, Fp[2] <- X2
  auto fwd_epi = [&](const OpT* b, f32x16 (&F)[3], f32x16 (&Fp)[3], const float* ebuf, auto EPI) {
    constexpr bool DO_EPI = decltype(EPI)::value;
    const int kro = th * 32 + (lane & 31), kco = (lane >> 5) * M::KSUB;
    const float* er = ebuf + th * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < 3; ++m) zero(F[m]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const auto kf = M::load(b + TL::at(kro, kco + s * M::KSTEP));
      F[0] = M::mma(kf, wf[0][s], F[0]);
      F[1] = M::mma(kf, wf[1][s], F[1]);
      if constexpr (!LINATTN) F[2] = M::mma(M::load(b + TILE + TL::at(kro, kco + s * M::KSTEP)), wf[2][s], F[2]);
      if constexpr (DO_EPI) {
#pragma unroll
        for (int r = 16 * s / KS; r < 16 * (s + 1) / KS; ++r) {
          const int ti = 8 * (r >> 2) + (r & 3);
          const float e = er[(E3 ? TT : 0) + ti];  // eta (eta_1 with E3)
          const float A = Fp[0][r], Bm = Fp[1][r];
          const float sg = sigmoid_fast(A);
          const float sil = A * sg;
          const float eB = e * Bm;
          Fp[0][r] = sil * eB;
          if constexpr (!LINATTN) {
            const float Dr = Fp[2][r];
            const float e0 = E3 ? er[ti] : e, e2 = E3 ? er[2 * TT + ti] : e;
            Fp[1][r] = ((E3 ? e0 * Bm : eB) * Dr) * (sg * fmaf(A, 1.f - sg, 1.f));
            Fp[2][r] = (e2 * sil) * Dr;
          }
        }
      }
    }
  };
  // token contractions of the tile in buffer `b`: own token half from registers, then the
  // partner's half from the exchange area; output columns (cb0 + cc) * 32..
  auto contract = [&](const OpT* b, const f32x16 (&F)[3]) {
    frag own[NMAT][QS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        own[m][q] = acc_to_afrag<OpT>(F[m], q);
        xch[((w * NMAT + m) * QS + q) * 64 + lane] = own[m][q];
      }
    __syncthreads();  // partner fragments published
    const frag* pf = xch + (size_t)(w ^ 2) * NMAT * QS * 64 + lane;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int hrow = (half == 0 ? th : 1 - th) * 32;  // token rows of this half
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        frag am[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) am[m] = half == 0 ? own[m][q] : pf[(m * QS + q) * 64];
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
          const int c = cb0 + cc;
          if (CB % 2 == 0 || c < CB) {
            // am[0] = eta H (with V) -> P1; am[1] = X0 (with K) -> P0; am[2] = X2 (with K) -> P2
            acc[0][cc] = M::mma(am[0], tile_kfrag_tr<TL>(b + TILE, hrow, c * 32, q, lane), acc[0][cc]);
            if constexpr (!LINATTN) {
              const auto bk = tile_kfrag_tr<TL>(b, hrow, c * 32, q, lane);
              acc[1][cc] = M::mma(am[1], bk, acc[1][cc]);
              acc[2][cc] = M::mma(am[2], bk, acc[2][cc]);
            }
          }
        }
      }
    }
  };
  // one pipeline step: publish tile i+1, prefetch tile i+2, forward(i+1) || epilogue(i),
  // contractions(i). At the last tile the forward reruns on the other buffer's stale (or unset)
  // contents and its result is discarded, which keeps the step free of branches.
  auto step = [&](int i, f32x16 (&Fc)[3], f32x16 (&Fn)[3]) {
    __syncthreads();  // every wave is done with buffer (i+1)&1 and the exchange area
    if (i + 1 < ntiles) {
      put(i + 1);
      if (i + 2 < ntiles) fetch(i + 2);
    }
    __syncthreads();  // tile i+1 published
    fwd_epi(tiles + ((i + 1) & 1) * 2 * TILE, Fn, Fc, eta_s + (i & 1) * NE * TT, std::true_type{});
    contract(tiles + (i & 1) * 2 * TILE, Fc);
  };

  if (ntiles > 0) {
    f32x16 F0[3], F1[3];
    put(0);
    if (ntiles > 1) fetch(1);
    __syncthreads();
    fwd_epi(tiles, F0, F1, eta_s, std::false_type{});
    for (int i = 0; i < ntiles; i += 2) {
      step(i, F0, F1);
      if (i + 1 < ntiles) step(i + 1, F1, F0);
    }
  }

  const float inv = 1.f / scale;
  float* ob = a.out + seg * a.out_y_stride + pair * a.out_pair_stride;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const int omat = LINATTN ? 0 : (m == 0 ? 1 : (m == 1 ? 0 : 2));
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int c = cb0 + cc;
      if (CB % 2 == 0 || c < CB) {
        float* o = ob + omat * a.out_mat_stride + ((int64_t)jb * RB + jh * 32) * H + c * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) o[acc_row(r, lane) * H + acc_col(lane)] = acc[m][cc][r] * inv;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// grad_ws_kernel: the LaCT partial sums P0, P1, P2 of grad_rd_kernel (same block mapping, same
// outputs) with the work of a workgroup split by role over 8 waves, so that every SIMD holds one
// wave of each role and the register file takes two waves per SIMD:
//   forward waves 0-3  (hidden half jh = w & 1, token half th = w >> 1 of a 64-token tile):
//       A = K W0, Bm = K W2, D = V W1^T from register-resident fast-weight fragments, then the
//       SwiGLU / silu' epilogue with the (scaled) step sizes; the three intermediates go to LDS
//       as contraction fragments;
//   contraction waves 4-7 (hidden half jh = w & 1, output columns (w >> 1 & 1)-th half):
//       the staging of the K / V tiles two steps ahead (global -> registers -> LDS, converted to
//       fp16), then P1 += (eta H)^T V, P0 += X0^T K, P2 += X2^T K over the tile.
// One barrier per step: the forward of tile i+1 runs beside the contraction of tile i, and each
// role orders its work so that its VALU phase meets the other role's MFMA phase.
template <class OpT, int H, bool E3 = false>
constexpr int grad_ws_lds_bytes() {
  return 3 * 2 * TT * TileLayout<OpT, H>::LD * (int)sizeof(OpT) + 3 * (E3 ? 3 : 1) * TT * 4 + 2 * 4 * 3 * 2 * 64 * 16;
}

// Workgroup index bid: XCD slot bid & 7; slot = bid >> 3 holds hidden block slot % njb of the
// (pair, segment) group (bid & 7) + 8 (slot / njb), group = pair * nseg + segment.
template <class IoT, class OpT, int H, bool SCALE_MID, bool E3 = false>
__device__ __forceinline__ void grad_ws_body(const GradArgs& a, int nseg, int npairs, int bid, unsigned char* smem) {
  constexpr int NE = E3 ? 3 : 1;  // step-size rows
  static_assert(std::is_same<OpT, _Float16>::value && (H == 64 || H == 128), "fp16 operands, h = 64 or 128");
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  typedef TileLayout<OpT, H> TL;
  typedef TileStage<IoT, OpT, H> Stage;
  constexpr int TILE = TT * TL::LD;         // elements of one staged tensor tile
  constexpr int CB = H / 32;
  constexpr int CH = CB / 2;                // output column blocks per contraction wave
  constexpr int KS = H / M::KSTEP;          // forward K steps over h
  constexpr int QS = 32 / M::KSTEP;         // contraction K steps over a 32-token half

  OpT* tiles = reinterpret_cast<OpT*>(smem);                      // [3 buffers][K, V][TT][LD]
  float* eta_s = reinterpret_cast<float*>(tiles + 3 * 2 * TILE);  // [3 buffers][NE][TT] scaled step sizes
  frag* inter = reinterpret_cast<frag*>(eta_s + 3 * NE * TT);     // [2][4 forward waves][3][QS][64]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int njb = a.rh / RB;
  const int xcd = bid & 7, slot = bid >> 3;
  const int jb = slot % njb;
  const int group = xcd + 8 * (slot / njb);
  if (group >= npairs * nseg) return;
  const int pair = group / nseg, seg = group % nseg;
  const int t_begin = a.t_base + seg * a.seg_len;
  const int t_end = min(t_begin + a.seg_len, a.t_limit);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + TT - 1) / TT : 0;
  const int jh = w & 1;

  const IoT* Kp = reinterpret_cast<const IoT*>(a.K) + pair * a.tok_pair_stride;
  const IoT* Vp = reinterpret_cast<const IoT*>(a.V) + pair * a.tok_pair_stride;
  const float* ep = a.eta + pair * a.eta_pair_stride;

  // requests first: fast weights (forward waves), tiles 0 and 1 and the segment's power-of-two
  // eta scale (contraction waves, the only users of the scale)
  const bool fwd = w < 4;
  const int ctid = tid - 256;
  frag wf[3][KS];
  Stage st0, st1;                           // staging registers of even / odd tiles
  float ev0 = 0.f, ev1 = 0.f;               // step size of token ctid of the staged tile
  auto fetch = [&](int i, Stage& stg, float& ev) {
    const int t0 = t_begin + i * TT;
    stg.load(Kp, Vp, t0, t_end, ctid);
    if (ctid < NE * TT) {
      const int e = ctid / TT, t = ctid % TT;
      ev = (t0 + t < t_end) ? ep[e * a.eta_mat_stride + t0 + t] : 0.f;
    }
  };
  if (fwd) {
    const OpT* src[3] = {reinterpret_cast<const OpT*>(a.W0T), reinterpret_cast<const OpT*>(a.W2T),
                         reinterpret_cast<const OpT*>(a.W1)};
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const OpT* row = src[m] + pair * a.w_pair_stride + (int64_t)(jb * RB + jh * 32 + (lane & 31)) * H +
                       (lane >> 5) * M::KSUB;
#pragma unroll
      for (int s = 0; s < KS; ++s) wf[m][s] = M::load(row + s * M::KSTEP);
    }
  } else if (ntiles > 0) {
    fetch(0, st0, ev0);
    if (ntiles > 1) fetch(1, st1, ev1);
  }
  float scale = 1.f;
  if constexpr (SCALE_MID) scale = a.eta_scale[pair * nseg + seg];

  if (fwd) {
    // ---------------- forward waves ----------------
    const int th = w >> 1;
    if (ntiles > 0) __syncthreads();  // tile 0 staged
    int fb = 0;                       // buffer of tile i + 1
    for (int i = -1; i < ntiles; ++i) {
      if (i + 1 < ntiles) {
        const OpT* b = tiles + fb * 2 * TILE;
        const int kro = th * 32 + (lane & 31), kco = (lane >> 5) * M::KSUB;
        f32x16 F[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) zero(F[m]);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const auto kf = M::load(b + TL::at(kro, kco + s * M::KSTEP));
          const auto vf = M::load(b + TILE + TL::at(kro, kco + s * M::KSTEP));
          F[0] = M::mma(kf, wf[0][s], F[0]);
          F[1] = M::mma(kf, wf[1][s], F[1]);
          F[2] = M::mma(vf, wf[2][s], F[2]);
        }
        // epilogue: F[0] <- eta*H, F[1] <- X0, F[2] <- X2, as contraction fragments
        const float* er = eta_s + fb * NE * TT + th * 32 + 4 * (lane >> 5);
        frag* dst = inter + (size_t)((((i + 1) & 1) * 4 + w) * 3) * QS * 64 + lane;
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          frag o0, o1, o2;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * q + e;
            const int ti = 8 * (r >> 2) + (r & 3);
            const float ev = er[(E3 ? TT : 0) + ti];  // eta (eta_1 with E3)
            const float A = F[0][r], Bm = F[1][r], Dr = F[2][r];
            const float sg = sigmoid_fast(A);
            const float sil = A * sg;
            const float eB = ev * Bm;
            o0[e] = M::from_f32(sil * eB);
            const float e0B = E3 ? er[ti] * Bm : eB;
            const float e2 = E3 ? er[2 * TT + ti] : ev;
            o1[e] = M::from_f32((e0B * Dr) * fmaf(sil, 1.f - sg, sg));  // silu'(A) = sg + silu(A) (1 - sg)
            o2[e] = M::from_f32((e2 * sil) * Dr);
          }
          dst[(0 * QS + q) * 64] = o0;
          dst[(1 * QS + q) * 64] = o1;
          dst[(2 * QS + q) * 64] = o2;
        }
      }
      fb = fb == 2 ? 0 : fb + 1;
      __syncthreads();
    }
    return;
  }

  // ---------------- contraction waves ----------------
  const int cpair = (w >> 1) & 1;           // output column blocks cpair * CH ..
  auto put = [&](int buf, const Stage& stg, float ev) {
    OpT* b = tiles + buf * 2 * TILE;
    stg.template store_at<TL>(b, b + TILE, ctid);
    if (ctid < NE * TT) eta_s[buf * NE * TT + ctid] = ev * scale;
  };

  f32x16 acc[3][CH];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int c = 0; c < CH; ++c) zero(acc[m][c]);

  if (ntiles > 0) {
    put(0, st0, ev0);
    if (ntiles > 2) fetch(2, st0, ev0);
    __syncthreads();  // tile 0 staged
  }
  int cb = 0;         // buffer of tile i (tile i + 2 goes to buffer cb + 2 mod 3)
  // step i: staging of tile i + 2 first (VALU and LDS writes, while the forward waves run their
  // MFMAs), then the contraction of tile i (while they run the epilogue). Tile t is staged from
  // register set t & 1, requested two steps before it is stored.
  auto step = [&](int i, Stage& stg, float& ev) {
    const int pb = cb == 0 ? 2 : cb - 1;    // buffer of tile i + 2 (= the buffer of tile i - 1)
    if (i + 2 < ntiles) {
      put(i < 0 ? 1 : pb, stg, ev);
      if (i + 4 < ntiles) fetch(i + 4, stg, ev);
    }
    if (i >= 0) {
      const OpT* b = tiles + cb * 2 * TILE;
      const frag* src = inter + (size_t)((i & 1) * 4 * 3) * QS * 64 + lane;
#pragma unroll
      for (int th2 = 0; th2 < 2; ++th2) {
        const frag* fsrc = src + (size_t)((jh + 2 * th2) * 3) * QS * 64;
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          frag am[3];
#pragma unroll
          for (int m = 0; m < 3; ++m) am[m] = fsrc[(m * QS + q) * 64];
#pragma unroll
          for (int cc = 0; cc < CH; ++cc) {
            const int c = cpair * CH + cc;
            // am[0] = eta H (with V) -> P1; am[1] = X0 (with K) -> P0; am[2] = X2 (with K) -> P2
            acc[0][cc] = M::mma(am[0], tile_kfrag_tr<TL>(b + TILE, 32 * th2, c * 32, q, lane), acc[0][cc]);
            const auto bk = tile_kfrag_tr<TL>(b, 32 * th2, c * 32, q, lane);
            acc[1][cc] = M::mma(am[1], bk, acc[1][cc]);
            acc[2][cc] = M::mma(am[2], bk, acc[2][cc]);
          }
        }
      }
    }
    if (i >= 0) cb = cb == 2 ? 0 : cb + 1;
    __syncthreads();
  };
  for (int i = -1; i < ntiles; i += 2) {
    step(i, st1, ev1);
    if (i + 1 < ntiles) step(i + 1, st0, ev0);
  }

  const float inv = 1.f / scale;
  float* ob = a.out + seg * a.out_y_stride + pair * a.out_pair_stride;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int omat = m == 0 ? 1 : (m == 1 ? 0 : 2);
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int c = cpair * CH + cc;
      float* o = ob + omat * a.out_mat_stride + ((int64_t)jb * RB + jh * 32) * H + c * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[acc_row(r, lane) * H + acc_col(lane)] = acc[m][cc][r] * inv;
    }
  }
}

template <class IoT, class OpT, int H, bool SCALE_MID, bool E3 = false>
__global__ void __launch_bounds__(512) grad_ws_kernel(GradArgs a, int nseg, int npairs) {
  extern __shared__ __align__(16) unsigned char smem[];
  grad_ws_body<IoT, OpT, H, SCALE_MID, E3>(a, nseg, npairs, blockIdx.x, smem);
}

// ------------------------------------------------------------------------------------------
struct ApplyArgs {
  const void* Q;            // [pair][Nq][H]
  int64_t tok_pair_stride;
  int t_base;               // first query token of the launch (a chunk boundary)
  int t_limit;              // one past the last query token of the launch
  int tiles_per_chunk;      // grid.x = chunks * tiles_per_chunk; tiles never straddle chunks
  const void* W0T;          // [rh][H] per pair
  const void* W2T;
  int64_t w_pair_stride;
  const void* W1T;          // [H][rh] per pair, optionally per chunk
  int64_t w1t_pair_stride;
  int64_t w1t_chunk_stride; // elements between chunks' W1T (0: one W1T for all tokens)
  int chunk;                // query tokens per chunk (selects the W1T of a query tile)
  int rh;
  void* O;                  // [pair][Nq][H]
  int npairs;               // pairs in the launch
  int ntiles;               // query tiles per pair in the launch (chunks * tiles_per_chunk)
  const void* W1;           // [rh][H] per pair (rows j), optionally per chunk (apply_rd_kernel)
  int64_t w1_pair_stride;
  int64_t w1_chunk_stride;
};

template <class OpT, int H>
constexpr int apply_lds_bytes() {
  constexpr int P = Pad<OpT>::v;
  return (TT * (H + P) + 2 * RB * (H + P) + H * (RB + P) + TT * (RB + P)) * (int)sizeof(OpT);
}

// grid: x = 8 * ceil(npairs / 8) * ntiles; all tiles of a pair run on one XCD (workgroups
// w, w+8, ...), so its fast-weight shadows stay in that XCD's L2. block: 256 threads.
template <class IoT, class OpT, int H>
__global__ void __launch_bounds__(256) apply_kernel(ApplyArgs a) {
  typedef Mfma<OpT> M;
  constexpr int P = Pad<OpT>::v;
  constexpr int LDQ = H + P, LDH = RB + P;
  constexpr int CB = H / 32;
  constexpr int NO = 2 * CB;                      // output tiles (2 token halves x CB)
  constexpr int NT = (NO + NWAVE - 1) / NWAVE;
  extern __shared__ __align__(16) unsigned char smem[];
  OpT* Qs = reinterpret_cast<OpT*>(smem);  // [TT][LDQ]
  OpT* W0s = Qs + TT * LDQ;                // [RB][LDQ]
  OpT* W2s = W0s + RB * LDQ;               // [RB][LDQ]
  OpT* W1s = W2s + RB * LDQ;               // [H][LDH]
  OpT* Hs = W1s + H * LDH;                 // [TT][LDH]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bid = blockIdx.x, slot = bid >> 3;
  const int pair = (bid & 7) + 8 * (slot / a.ntiles);
  const int tile = slot % a.ntiles;
  if (pair >= a.npairs) return;
  const int chunk_idx = tile / a.tiles_per_chunk;
  const int t0 = a.t_base + chunk_idx * a.chunk + (tile % a.tiles_per_chunk) * TT;
  const int t_lim = min(a.t_base + (chunk_idx + 1) * a.chunk, a.t_limit);
  if (t0 >= t_lim) return;
  const IoT* Qp = reinterpret_cast<const IoT*>(a.Q) + pair * a.tok_pair_stride;
  const OpT* w0g = reinterpret_cast<const OpT*>(a.W0T) + pair * a.w_pair_stride;
  const OpT* w2g = reinterpret_cast<const OpT*>(a.W2T) + pair * a.w_pair_stride;
  const OpT* w1g = reinterpret_cast<const OpT*>(a.W1T) + pair * a.w1t_pair_stride +
                   (int64_t)chunk_idx * a.w1t_chunk_stride;

  // stage the query tile (converted to the operand type); rows beyond the limit are zero
  {
    constexpr int VE = Io<IoT>::VEC;
    for (int i = tid; i < TT * H / VE; i += 256) {
      const int row = i / (H / VE), c = (i % (H / VE)) * VE;
      OpT tmp[VE];
      if (t0 + row < t_lim) {
        Io<IoT>::template load_cvt<OpT>(Qp + (int64_t)(t0 + row) * H + c, tmp);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) tmp[e] = M::from_f32(0.f);
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) Qs[row * LDQ + c + e] = tmp[e];
    }
  }
  f32x16 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) zero(acc[i]);

  const int th = w >> 1, jh = w & 1;
  constexpr int VW = 16 / sizeof(OpT);
  for (int j0 = 0; j0 < a.rh; j0 += RB) {
    __syncthreads();
    for (int i = tid; i < RB * H / VW; i += 256) {
      const int row = i / (H / VW), c = (i % (H / VW)) * VW;
      *reinterpret_cast<u32x4*>(W0s + row * LDQ + c) =
          *reinterpret_cast<const u32x4*>(w0g + (int64_t)(j0 + row) * H + c);
      *reinterpret_cast<u32x4*>(W2s + row * LDQ + c) =
          *reinterpret_cast<const u32x4*>(w2g + (int64_t)(j0 + row) * H + c);
    }
    for (int i = tid; i < H * RB / VW; i += 256) {
      const int row = i / (RB / VW), c = (i % (RB / VW)) * VW;
      *reinterpret_cast<u32x4*>(W1s + row * LDH + c) =
          *reinterpret_cast<const u32x4*>(w1g + (int64_t)row * a.rh + j0 + c);
    }
    __syncthreads();
    // hidden activations for tokens th*32.., hidden units jh*32..
    {
      f32x16 fa, fb;
      zero(fa);
      zero(fb);
      mma_tile<OpT, H>(fa, Qs + th * 32 * LDQ, LDQ, W0s + jh * 32 * LDQ, LDQ, lane);
      mma_tile<OpT, H>(fb, Qs + th * 32 * LDQ, LDQ, W2s + jh * 32 * LDQ, LDQ, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float A = fa[r];
        const float hv = A * sigmoidf_(A) * fb[r];
        Hs[(th * 32 + acc_row(r, lane)) * LDH + jh * 32 + acc_col(lane)] = M::from_f32(hv);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int q = w + NWAVE * i;
      if (q < NO) {
        const int tq = q % 2, cb = q / 2;
        mma_tile<OpT, RB>(acc[i], Hs + tq * 32 * LDH, LDH, W1s + cb * 32 * LDH, LDH, lane);
      }
    }
  }
  IoT* Op = reinterpret_cast<IoT*>(a.O) + pair * a.tok_pair_stride;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int q = w + NWAVE * i;
    if (q < NO) {
      const int tq = q % 2, cb = q / 2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + tq * 32 + acc_row(r, lane);
        if (t < t_lim) Io<IoT>::store(Op + (int64_t)t * H + cb * 32 + acc_col(lane), acc[i][r]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Register-direct apply for h <= 128: a workgroup of 8 waves takes AT = 256 query tokens of one
// pair, wave w the 32 tokens t0 + 32 w .. Its query rows stay in registers as MFMA B fragments
// for the whole launch; the fast weights stream through LDS in blocks of AJ = 64 hidden units
// (W0^T, W2^T and W1 rows, double-buffered in LDS, each block requested two blocks ahead
// through two alternating register sets, shared by the 8 waves). Per 32-unit half of a block
// the wave forms C0[j][t] = W0^T Q^T and C2[j][t] = W2^T Q^T (hidden rows as the A operand);
// the SwiGLU values h = silu(C0) * C2 become the A fragments of O[t][c] += sum_j h[t][j] W1[j][c]
// directly (acc_to_afrag), and W1's rows are read K-major through the permuted transpose read
// (acc_kfrag_tr). No activation tile goes through LDS.
// grid: x = 8 * ceil(npairs / 8) * ntiles (all tiles of a pair on one XCD); block 512.
constexpr int AT = 256;
constexpr int AJ = 64;

template <class OpT>
constexpr int tr_ld(int cols) {  // row stride for transpose reads of 16-bit rows without bank conflicts
  if (sizeof(OpT) != 2) return cols + 4;
  int l = cols + 4;
  while ((l / 2) % 32 != 16) l += 4;
  return l;
}

template <class OpT, int H>
struct ApplyRdLayout {
  static constexpr int LDW = H + Pad<OpT>::v;       // W0^T / W2^T block rows
  static constexpr int LD1 = tr_ld<OpT>(H);        // W1 block rows (transpose reads)
  static constexpr int BUF = (2 * AJ * LDW + AJ * LD1) * (int)sizeof(OpT);
  static constexpr int bytes = 2 * BUF;
};

template <class OpT, int H>
constexpr int apply_rd_lds_bytes() { return ApplyRdLayout<OpT, H>::bytes; }

template <class IoT, class OpT, int H>
__device__ __forceinline__ void apply_rd_body(const ApplyArgs& a, int bid, unsigned char* smem) {
  static_assert(H <= 128, "register budget");
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  typedef ApplyRdLayout<OpT, H> L;
  constexpr int LDW = L::LDW, LD1 = L::LD1;
  constexpr int KS = H / M::KSTEP;          // K steps over h
  constexpr int QS = 32 / M::KSTEP;         // K steps over a 32-unit hidden half block
  constexpr int CB = H / 32;
  constexpr int VW = 16 / (int)sizeof(OpT); // elements per 16-byte chunk
  constexpr int NCPM = AJ * H / VW;         // 16-byte chunks of one matrix's slice
  constexpr int NCHK = 3 * NCPM;            // 16-byte chunks of one staged block
  constexpr int CPT = (NCHK + 511) / 512;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = bid >> 3;
  const int pair = (bid & 7) + 8 * (slot / a.ntiles);
  const int tile = slot % a.ntiles;
  if (pair >= a.npairs) return;
  const int chunk_idx = tile / a.tiles_per_chunk;
  const int t0 = a.t_base + chunk_idx * a.chunk + (tile % a.tiles_per_chunk) * AT;
  const int t_lim = min(a.t_base + (chunk_idx + 1) * a.chunk, a.t_limit);
  if (t0 >= t_lim) return;
  const int tw = t0 + 32 * w;               // this wave's first token

  const IoT* Qp = reinterpret_cast<const IoT*>(a.Q) + pair * a.tok_pair_stride;
  const OpT* w0g = reinterpret_cast<const OpT*>(a.W0T) + pair * a.w_pair_stride;
  const OpT* w2g = reinterpret_cast<const OpT*>(a.W2T) + pair * a.w_pair_stride;
  const OpT* w1g = reinterpret_cast<const OpT*>(a.W1) + pair * a.w1_pair_stride +
                   (int64_t)chunk_idx * a.w1_chunk_stride;
  const int njb = a.rh / AJ;

  // staged block jb: rows jb*AJ .. of W0^T, W2^T, W1 (16-byte chunks, plain copies)
  u32x4 sva[CPT], svb[CPT];
  auto bufp = [&](int i) { return reinterpret_cast<OpT*>(smem + (i & 1) * L::BUF); };
  auto load_blk = [&](int jb, u32x4 (&sv)[CPT]) {
    if (jb >= njb) return;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + 512 * i;
      if (NCHK % 512 == 0 || ch < NCHK) {
        // matrix of chunk i: a compile-time constant when every 512-chunk step stays in one matrix
        const int m = NCPM % 512 == 0 ? 512 * i / NCPM : ch / NCPM;
        const int r = (ch / (H / VW)) % AJ, c = (ch % (H / VW)) * VW;
        const OpT* src = (m == 0 ? w0g : m == 1 ? w2g : w1g) + (int64_t)(jb * AJ + r) * H + c;
        sv[i] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };
  auto store_blk = [&](OpT* b, const u32x4 (&sv)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + 512 * i;
      if (NCHK % 512 == 0 || ch < NCHK) {
        const int m = NCPM % 512 == 0 ? 512 * i / NCPM : ch / NCPM;
        const int r = (ch / (H / VW)) % AJ, c = (ch % (H / VW)) * VW;
        OpT* dst = m < 2 ? b + m * AJ * LDW + r * LDW + c : b + 2 * AJ * LDW + r * LD1 + c;
        *reinterpret_cast<u32x4*>(dst) = sv[i];
      }
    }
  };

  load_blk(0, sva);
  load_blk(1, svb);

  // query rows as B fragments: lane (n = token lane & 31, k = c); rows past the limit are zero
  frag qf[KS];
  {
    const int t = tw + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      OpT tmp[M::KSUB];
      const int c = s * M::KSTEP + (lane >> 5) * M::KSUB;
      if (t < t_lim) {
        if constexpr (M::KSUB == 8) {
          Io<IoT>::template load_cvt<OpT>(Qp + (int64_t)t * H + c, tmp);
        } else {
          static_assert(std::is_same<IoT, float>::value, "fp32 operands come with fp32 I/O");
          tmp[0] = Qp[(int64_t)t * H + c];
        }
      } else {
#pragma unroll
        for (int e = 0; e < M::KSUB; ++e) tmp[e] = M::from_f32(0.f);
      }
      if constexpr (M::KSUB == 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = tmp[e];
      } else {
        qf[s] = tmp[0];
      }
    }
  }

  store_blk(bufp(0), sva);
  load_blk(2, sva);
  __syncthreads();

  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) zero(o[cb]);

  // block jb: publish block jb+1 (requested two blocks ago), request block jb+3, compute jb
  auto step = [&](int jb, u32x4 (&nxt)[CPT]) {
    if (jb + 1 < njb) store_blk(bufp(jb + 1), nxt);
    load_blk(jb + 3, nxt);
    const OpT* b = bufp(jb);
    if (tw < t_lim) {
#pragma unroll
      for (int hb = 0; hb < AJ / 32; ++hb) {
        f32x16 c0, c2;
        zero(c0);
        zero(c2);
        const OpT* r0 = b + (hb * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
        const OpT* r2 = r0 + AJ * LDW;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          c0 = M::mma(M::load(r0 + s * M::KSTEP), qf[s], c0);
          c2 = M::mma(M::load(r2 + s * M::KSTEP), qf[s], c2);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float A = c0[r];
          c0[r] = A * sigmoid_fast(A) * c2[r];
        }
        const OpT* w1s = b + 2 * AJ * LDW + hb * 32 * LD1;
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          const frag hf = acc_to_afrag<OpT>(c0, q);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            o[cb] = M::mma(hf, acc_kfrag_tr<OpT>(w1s + cb * 32, LD1, q, lane), o[cb]);
        }
      }
    }
    __syncthreads();
  };
  for (int jb = 0; jb < njb; jb += 2) {
    step(jb, svb);
    if (jb + 1 < njb) step(jb + 1, sva);
  }

  if (tw < t_lim) {
    IoT* Op = reinterpret_cast<IoT*>(a.O) + pair * a.tok_pair_stride;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tw + acc_row(r, lane);
        if (t < t_lim) Io<IoT>::store(Op + (int64_t)t * H + cb * 32 + acc_col(lane), o[cb][r]);
      }
  }
}

// workgroup bid: pair (bid & 7) + 8 * (slot / ntiles), 256-token tile slot % ntiles (slot = bid >> 3)
template <class IoT, class OpT, int H>
__global__ void __launch_bounds__(512) apply_rd_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  apply_rd_body<IoT, OpT, H>(a, blockIdx.x, smem);
}

}  // namespace ttt
