// linattn_fused.hpp -- single-pass linear-attention form on gfx950 (rh <= 128).
//
// With only W1 written and no renormalisation the fast weight's kernel phi(x) = silu(x W0) * (x W2)
// is static and the state update is associative (KV-binding summary page, "Prerequisites ->
// Linear attention" and Theorem 5.2 under "Method step details"; press article, section 4):
//   dS_c = phi(K_c)^T diag(eta_c) V_c,   S_c = W1 + sum_{j<c} dS_j (apply-then-update; j <= c for
//   update-then-apply),   O_c = phi(Q_c) S_c.
// One launch, one workgroup per (pair, group of G consecutive chunks); a group behaves as one
// chunk of G*chunk tokens for the scan (its aggregate is the sum of its chunks' aggregates, added
// in chunk order) while each chunk's queries still read their own state:
//   A. the chunk aggregate dS_c from K_c, V_c, eta_c (hidden-row ownership: wave (jb, th) holds
//      W0^T / W2^T rows jb*32.. as MFMA fragments and sums its token half; halves combined in a
//      fixed order), published to L2 with a flag;
//   B. decoupled lookback over the pair's chunk states: walk back to the nearest published
//      inclusive prefix (or to W1 at the start of the sequence), add the aggregates after it left
//      to right, publish the inclusive prefix. Every inclusive prefix is the same left-to-right sum
//      W1 + dS_0 + dS_1 + ..., so the result is bitwise independent of where the walk stopped;
//   C. O_c = phi(Q_c) S_c (token ownership: wave w takes 32 query tokens, the fast weights and
//      S_c are read from LDS).
// Q, K, V are read once and O written once: the compulsory traffic of the form.
//
// Cross-workgroup visibility: all chunks of a pair run on one XCD, whose L2 is the point of
// coherence. A writer drains its stores (s_waitcnt vmcnt(0)) before a relaxed device-scope flag
// store; readers poll the flag with device-scope loads and read the data with device-scope loads,
// which miss in the per-CU L1. Forward progress: a workgroup takes a ticket from its XCD's counter
// (hardware XCC id) and works on the ticket-th (pair, chunk) of that XCD in chunk order, so every
// predecessor it may wait for holds a smaller ticket, i.e. has started. Waits are bounded; a timeout
// raises the error word and the chunk's outputs are written as NaN.
#pragma once
#include "fastweight.hpp"

namespace ttt {

struct FusedArgs {
  const void* Q;            // [pair][N][H] I/O type
  const void* K;
  const void* V;
  const float* eta;         // [pair][N]
  const float* W0;          // row form [b][h][rh] (w_batch_stride between sequences; 0 = shared)
  const float* W2;
  const float* W1;          // [b][rh][h]
  void* O;                  // [pair][N][H]
  float* S_out;             // [pair][rh][h] final state, or null
  float* agg;               // [pair][nch][rh*h] chunk aggregates (workspace)
  float* incl;              // [pair][nch][rh*h] inclusive prefixes (workspace)
  unsigned* flags;          // [pair][nch]: 1 aggregate published, 2 inclusive prefix published
  unsigned* tickets;        // [8] per-XCD work counters, then the error word at [8]
  int P, heads, N, chunk, nch, inclusive;
  int group;                // chunks per workgroup G (nch % G == 0; G > 1 needs chunk % (NW*32) == 0)
  int64_t w_batch_stride;
};

constexpr long FUSED_SPIN_LIMIT = 1l << 20;

__device__ __forceinline__ unsigned hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15;  // HW_REG_XCC_ID[3:0]
}
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned flag_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte loads with the device-scope cache policy (sc1: miss in the per-CU L1, read the XCD's
// L2) through a raw buffer resource over [base, base + bytes); out-of-range offsets read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 dev_load4(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 16);
}

// zero the tickets, the error word and the flags before a launch. grid 1, block 256.
__global__ void __launch_bounds__(256) linattn_fused_reset(unsigned* tickets, unsigned* flags, int nflags) {
  if (threadIdx.x < 9) tickets[threadIdx.x] = 0u;
  for (int i = threadIdx.x; i < nflags; i += 256) flags[i] = 0u;
}

template <class OpT, int H, int RH>
struct FusedLayout {
  static constexpr int NJB = RH / 32, NW = 2 * NJB, NT = 64 * NW;
  static constexpr int LDK = H + Pad<OpT>::v;       // token tiles (row reads and transpose reads)
  static constexpr int LDW = H + Pad<OpT>::v;       // W0^T / W2^T rows
  static constexpr int LD1 = tr_ld<OpT>(H);         // S rows (transpose reads)
  static constexpr int TILE = TT * LDK;             // elements of one staged token tile
  static constexpr int TILES_B = 4 * TILE * (int)sizeof(OpT);                 // 2 buffers x (K, V)
  static constexpr int COMB_B = NJB * 32 * H * 4;                            // token-half combine
  static constexpr int OST_B = NW * 32 * (H + 8) * 2;                         // output staging
  static constexpr int R0 = TILES_B > COMB_B ? (TILES_B > OST_B ? TILES_B : OST_B) : (COMB_B > OST_B ? COMB_B : OST_B);
  static constexpr int ETA_O = R0;                                           // [2][TT] floats
  static constexpr int WT_O = ETA_O + 2 * TT * 4;                            // W0^T, W2^T [RH][LDW]
  static constexpr int SS_O = WT_O + 2 * RH * LDW * (int)sizeof(OpT);        // S [RH][LD1]
  static constexpr int bytes = SS_O + RH * LD1 * (int)sizeof(OpT) + 16;
};

template <class OpT, int H, int RH>
constexpr int linattn_fused_lds_bytes() { return FusedLayout<OpT, H, RH>::bytes; }

// grid: 8 * ceil(P / 8) * (nch / G) workgroups; block NT = 128 * RH / 32 threads.
template <class IoT, class OpT, int H, int RH>
__global__ void __launch_bounds__(128 * (RH / 32)) linattn_fused_kernel(FusedArgs a) {
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  typedef FusedLayout<OpT, H, RH> L;
  constexpr int NJB = L::NJB, NW = L::NW, NT = L::NT;
  constexpr int LDK = L::LDK, LDW = L::LDW, LD1 = L::LD1, TILE = L::TILE;
  constexpr int KS = H / M::KSTEP;          // K steps over h
  constexpr int QS = 32 / M::KSTEP;         // K steps over 32 tokens / 32 hidden units
  constexpr int CB = H / 32;                // 32-column blocks of h
  constexpr int VE = Io<IoT>::VEC;          // I/O elements per 16-byte chunk
  constexpr int NCK = TT * H / VE;          // 16-byte chunks of one token tile
  constexpr int CPT = (NCK + NT - 1) / NT;
  constexpr int NS4 = RH * H / 4;           // float4 groups of the state
  constexpr int SPT = (NS4 + NT - 1) / NT;
  static_assert(RH % 32 == 0 && H % 32 == 0 && NT <= 1024, "shape");

  extern __shared__ __align__(16) unsigned char smem[];
  OpT* tiles = reinterpret_cast<OpT*>(smem);                       // [2][K, V][TT][LDK]
  float* comb = reinterpret_cast<float*>(smem);                    // phase A combine (after tiles)
  bf16_t* ost = reinterpret_cast<bf16_t*>(smem);                   // phase C output staging
  float* eta_s = reinterpret_cast<float*>(smem + L::ETA_O);        // [2][TT]
  OpT* Wt = reinterpret_cast<OpT*>(smem + L::WT_O);                // [2][RH][LDW]
  OpT* Ss = reinterpret_cast<OpT*>(smem + L::SS_O);                // [RH][LD1]
  int* ctl = reinterpret_cast<int*>(smem + L::bytes - 16);         // ticket, stop, bad

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    const unsigned x = hw_xcc_id();
    const unsigned t = __hip_atomic_fetch_add(a.tickets + (x & 7), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ctl[0] = (int)t;
    ctl[1] = (int)(x & 7);
    ctl[2] = 0;
  }
  __syncthreads();
  const int ticket = ctl[0], xcd = ctl[1];
  const int G = a.group, ngr = a.nch / G;
  const int pair = xcd + 8 * (ticket / ngr), ch = ticket % ngr;  // ch: the group's index
  if (pair >= a.P) return;
  const int64_t n = (int64_t)RH * H;
  const int cbase = ch * G * a.chunk, cend = cbase + G * a.chunk;  // the group's tokens
  const int b = pair / a.heads, head = pair % a.heads;
  const float* W0p = a.W0 + (int64_t)b * a.w_batch_stride + (int64_t)head * n;  // [h][rh]
  const float* W2p = a.W2 + (int64_t)b * a.w_batch_stride + (int64_t)head * n;
  const float* W1p = a.W1 + (int64_t)b * a.w_batch_stride + (int64_t)head * n;  // [rh][h]
  const IoT* Kp = reinterpret_cast<const IoT*>(a.K) + (int64_t)pair * a.N * H;
  const IoT* Vp = reinterpret_cast<const IoT*>(a.V) + (int64_t)pair * a.N * H;
  const IoT* Qp = reinterpret_cast<const IoT*>(a.Q) + (int64_t)pair * a.N * H;
  const float* ep = a.eta + (int64_t)pair * a.N;
  unsigned* fl = a.flags + (int64_t)pair * a.nch;
  float* aggp = a.agg + (int64_t)pair * a.nch * n;
  float* inclp = a.incl + (int64_t)pair * a.nch * n;

  // ---- token-tile staging of K, V, eta (rows past the chunk end are zero); NPF register sets
  // rotate, so a tile is requested NPF tiles before it is stored to LDS ----
  struct Staged {
    u32x4 k[CPT], v[CPT];
    float e;
  };
  constexpr int NPF = 4;
  Staged sg4[NPF];
  auto fetch = [&](int t0, Staged& sg) {
    u32x4* sk = sg.k;
    u32x4* sv = sg.v;
    if (t0 >= cend) return;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c16 = tid + NT * i;
      const int row = c16 / (H / VE), col = (c16 % (H / VE)) * VE;
      const bool in = (NCK % NT == 0 || c16 < NCK) && t0 + row < cend;
      sk[i] = in ? *reinterpret_cast<const u32x4*>(Kp + (int64_t)(t0 + row) * H + col) : u32x4{0u, 0u, 0u, 0u};
      sv[i] = in ? *reinterpret_cast<const u32x4*>(Vp + (int64_t)(t0 + row) * H + col) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < TT) sg.e = (t0 + tid < cend) ? ep[t0 + tid] : 0.f;
  };
  auto put = [&](int buf, const Staged& sg) {
    const u32x4* sk = sg.k;
    const u32x4* sv = sg.v;
    OpT* kb = tiles + buf * 2 * TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c16 = tid + NT * i;
      if (NCK % NT == 0 || c16 < NCK) {
        const int row = c16 / (H / VE), col = (c16 % (H / VE)) * VE;
        TileStage<IoT, OpT, H>::put(sk[i], kb + row * LDK + col);
        TileStage<IoT, OpT, H>::put(sv[i], kb + TILE + row * LDK + col);
      }
    }
    if (tid < TT) eta_s[buf * TT + tid] = sg.e;
  };

  const int ntile = (G * a.chunk + TT - 1) / TT;
#pragma unroll
  for (int k = 0; k < NPF; ++k) fetch(cbase + k * TT, sg4[k]);

  // ---- fast-weight fragments of hidden rows jb*32 + (lane & 31): MFMA B operands in phase A,
  // A operands in phase C (same lane layout); W0^T / W2^T also go to LDS for phase C ----
  const int jb = w % NJB, th = w / NJB;
  frag wf[2][KS];
  {
    const int j = jb * 32 + (lane & 31);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* src = m == 0 ? W0p : W2p;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k0 = s * M::KSTEP + (lane >> 5) * M::KSUB;
        if constexpr (M::KSUB == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) wf[m][s][e] = M::from_f32(src[(int64_t)(k0 + e) * RH + j]);
          if (th == 0) *reinterpret_cast<frag*>(Wt + (m * RH + j) * LDW + k0) = wf[m][s];
        } else {
          wf[m][s] = src[(int64_t)k0 * RH + j];
          if (th == 0) Wt[(m * RH + j) * LDW + k0] = wf[m][s];
        }
      }
    }
  }

  // ---- A. chunk aggregate dS = phi(K)^T diag(eta) V ----
  f32x16 acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) zero(acc[c]);
  auto tile_step = [&](int i, Staged& sg) {
    __syncthreads();  // the buffer written next is no longer read
    put(i & 1, sg);
    fetch(cbase + (i + NPF) * TT, sg);
    __syncthreads();
    const OpT* kb = tiles + (i & 1) * 2 * TILE;
    const OpT* vb = kb + TILE;
    const float* es = eta_s + (i & 1) * TT;
    f32x16 fa, fb;
    zero(fa);
    zero(fb);
    const OpT* kr = kb + (th * 32 + (lane & 31)) * LDK + (lane >> 5) * M::KSUB;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const frag kf = M::load(kr + s * M::KSTEP);
      fa = M::mma(kf, wf[0][s], fa);
      fb = M::mma(kf, wf[1][s], fb);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float A = fa[r];
      fa[r] = es[th * 32 + acc_row(r, lane)] * (A * sigmoid_fast(A)) * fb[r];
    }
    const OpT* vh = vb + th * 32 * LDK;
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const frag af = acc_to_afrag<OpT>(fa, q);
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[c] = M::mma(af, acc_kfrag_tr<OpT>(vh + c * 32, LDK, q, lane), acc[c]);
    }
  };
  // token halves: wave (jb, 1) hands its sums to wave (jb, 0), which adds them in a fixed order.
  // Chunk i of the group: aggregate to slot ch*G + i for i < G-1; the group's sum (the chunks'
  // aggregates added in order) to slot ch*G + G-1. The combine area overlays the token tiles, whose
  // buffers are both free between the chunk's last step and the next step's store.
  f32x16 tot[CB];
  auto combine = [&](int i) {
    __syncthreads();
    if (th == 1) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) comb[((jb * CB + c) * 16 + r) * 64 + lane] = acc[c][r];
    }
    __syncthreads();
    if (th == 0) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[c][r] + comb[((jb * CB + c) * 16 + r) * 64 + lane];
          tot[c][r] = i == 0 ? v : tot[c][r] + v;
          acc[c][r] = v;
        }
      if (i < G - 1) {
        float* ag = aggp + ((int64_t)ch * G + i) * n + (int64_t)jb * 32 * H;
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) ag[acc_row(r, lane) * H + c * 32 + acc_col(lane)] = acc[c][r];
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) zero(acc[c]);
  };
  const int tpc = a.chunk / TT;  // tiles per chunk (G > 1: whole tiles)
  for (int i = 0; i < ntile; i += NPF) {
#pragma unroll
    for (int k = 0; k < NPF; ++k)
      if (i + k < ntile) {
        tile_step(i + k, sg4[k]);
        if (G > 1 && (i + k + 1) % tpc == 0 && i + k + 1 < ntile) combine((i + k) / tpc);
      }
  }
  combine(G - 1);
  if (th == 0) {
    float* ag = aggp + ((int64_t)ch * G + G - 1) * n + (int64_t)jb * 32 * H;
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) ag[acc_row(r, lane) * H + c * 32 + acc_col(lane)] = tot[c][r];
  }
  drain_stores();
  __syncthreads();
  if (tid == 0) __hip_atomic_store(fl + ch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // the first query pass's rows are requested now and arrive during the lookback
  static_assert(std::is_same<IoT, bf16_t>::value && std::is_same<OpT, _Float16>::value, "bf16 I/O");
  u32x4 qa[KS], qb[KS];
  auto load_q = [&](int t0, u32x4 (&qr)[KS]) {
    const int t = t0 + 32 * w + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = s * M::KSTEP + (lane >> 5) * M::KSUB;
      qr[s] = (t0 < cend && t < cend) ? *reinterpret_cast<const u32x4*>(Qp + (int64_t)t * H + c) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load_q(cbase, qa);

  // ---- B. decoupled lookback: wave 0 reads the flags of up to 64 predecessors at once (lane l:
  // chunk base - l); the nearest inclusive prefix ends the walk, a zero flag (aggregate not yet
  // published) is polled again, within a bounded number of polls ----
  if (w == 0) {
    int stop = -1, bad = 0;
    long spins = 0;
    for (int base = ch - 1; base >= 0;) {
      const int j = base - lane;
      const unsigned f = j >= 0 ? flag_load(fl + j) : 1u;
      const unsigned long long inc = __ballot(f == 2u), zero = __ballot(f == 0u);
      const int first2 = inc ? __builtin_ctzll(inc) : 64;               // nearest inclusive prefix
      const unsigned long long below = first2 >= 64 ? ~0ull : ((1ull << first2) - 1ull);
      if (zero & below) {                                              // an aggregate still missing
        if (++spins > FUSED_SPIN_LIMIT) {
          bad = 1;
          break;
        }
        continue;
      }
      if (first2 < 64) {
        stop = base - first2;
        break;
      }
      base -= 64;
    }
    if (lane == 0) {
      if (bad) __hip_atomic_fetch_add(a.tickets + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ctl[1] = stop;
      ctl[2] = bad;
    }
  }
  __syncthreads();
  const int stop = ctl[1];
  const bool bad = ctl[2] != 0;
  const __amdgpu_buffer_rsrc_t ra = dev_rsrc(aggp, (int)(a.nch * n * 4));
  const __amdgpu_buffer_rsrc_t ri = dev_rsrc(inclp, (int)(a.nch * n * 4));
  f32x4 run[SPT], ginc[SPT];  // state before the group's current chunk; the group's inclusive prefix
  {
    // prefix = (inclusive prefix at `stop`, or W1) + aggregates stop+1 .. ch-1, left to right;
    // loads of eight aggregates are in flight together
    f32x4 s[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      s[i] = stop >= 0 ? dev_load4(ri, (int)((stop * n + e) * 4)) : *reinterpret_cast<const f32x4*>(W1p + e);
    }
    for (int j0 = stop + 1; j0 < ch; j0 += 8) {
      f32x4 t[8][SPT];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
          const int e = 4 * (tid + NT * i);
          t[jj][i] = (j0 + jj < ch) ? dev_load4(ra, (int)((((j0 + jj) * G + G - 1) * n + e) * 4))
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < ch)
#pragma unroll
          for (int i = 0; i < SPT; ++i) s[i] += t[jj][i];
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      const f32x4 inc = s[i] + dev_load4(ra, (int)(((ch * G + G - 1) * n + e) * 4));
      *reinterpret_cast<f32x4*>(inclp + (int64_t)ch * n + e) = inc;
      if (ch == ngr - 1 && a.S_out) *reinterpret_cast<f32x4*>(a.S_out + (int64_t)pair * n + e) = inc;
      run[i] = s[i];
      ginc[i] = inc;
    }
  }
  drain_stores();
  __syncthreads();
  if (tid == 0) __hip_atomic_store(fl + ch, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- C. O = phi(Q) S for the chunk's query tokens, wave w: 32 tokens per pass ----
  const float poison = bad ? __builtin_nanf("") : 0.f;
  int oend = cend;  // end of the chunk whose outputs are written
  auto pass = [&](int t0, const u32x4 (&qcur)[KS], u32x4 (&qnext)[KS]) {
    load_q(t0 + NW * 32, qnext);
    const int tw = t0 + 32 * w;
    if (tw < oend) {
      frag qf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = bf16x8_to_f16x8(qcur[s]);
      f32x16 o[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) zero(o[c]);
#pragma unroll
      for (int j2 = 0; j2 < NJB; ++j2) {
        f32x16 c0, c2;
        zero(c0);
        zero(c2);
        const OpT* r0 = Wt + (j2 * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
        const OpT* r2 = r0 + RH * LDW;
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
        const OpT* sr = Ss + j2 * 32 * LD1;
#pragma unroll
        for (int q = 0; q < QS; ++q) {
          const frag hf = acc_to_afrag<OpT>(c0, q);
#pragma unroll
          for (int c = 0; c < CB; ++c) o[c] = M::mma(hf, acc_kfrag_tr<OpT>(sr + c * 32, LD1, q, lane), o[c]);
        }
      }
      // stage the wave's 32 x h output tile in LDS, then write whole 16-byte runs
      if constexpr (sizeof(IoT) == 2) {
        bf16_t* os = ost + w * 32 * (H + 8);
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) os[acc_row(r, lane) * (H + 8) + c * 32 + acc_col(lane)].bits = f32_to_bf16(o[c][r] + poison);
        IoT* Op = reinterpret_cast<IoT*>(a.O) + (int64_t)pair * a.N * H;
#pragma unroll
        for (int i = lane; i < 32 * H / 8; i += 64) {
          const int row = i / (H / 8), col = (i % (H / 8)) * 8;
          if (tw + row < oend)
            *reinterpret_cast<u32x4*>(Op + (int64_t)(tw + row) * H + col) =
                *reinterpret_cast<const u32x4*>(os + row * (H + 8) + col);
        }
      } else {
        IoT* Op = reinterpret_cast<IoT*>(a.O) + (int64_t)pair * a.N * H;
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tt = tw + acc_row(r, lane);
            if (tt < oend) Io<IoT>::store(Op + (int64_t)tt * H + c * 32 + acc_col(lane), o[c][r] + poison);
          }
      }
    }
  };
  // chunk i of the group reads S = run (+ its own aggregate when inclusive); run then advances by
  // the chunk's aggregate (the last chunk's inclusive state is the group's inclusive prefix)
  int np = 0;  // passes so far: even passes read qa and prefetch into qb, odd ones the reverse
  for (int i = 0; i < G; ++i) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int e = 4 * (tid + NT * k);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      const f32x4 nxt = i == G - 1 ? ginc[k] : run[k] + dev_load4(ra, (int)(((ch * G + i) * n + e) * 4));
      const f32x4 sc = a.inclusive ? nxt : run[k];
      const int j = e / H, c = e % H;
#pragma unroll
      for (int q = 0; q < 4; ++q) Ss[j * LD1 + c + q] = M::from_f32(sc[q]);
      run[k] = nxt;
    }
    __syncthreads();  // S of chunk i in LDS
    const int c0 = cbase + i * a.chunk;
    oend = c0 + a.chunk;
    for (int t0 = c0; t0 < oend; t0 += NW * 32, ++np) {
      if (np & 1)
        pass(t0, qb, qa);
      else
        pass(t0, qa, qb);
    }
    __syncthreads();  // every wave is done with S before the next chunk's is stored
  }
}

}  // namespace ttt
