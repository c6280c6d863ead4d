// linattn_fused.hpp -- single-pass linear-attention form on gfx950 (rh <= 128).
//
// With only W1 written and no renormalisation the fast weight's kernel phi(x) = silu(x W0) * (x W2)
// is static and the state update is associative (KV-binding summary page, "Prerequisites ->
// Linear attention" and Theorem 5.2 under "Method step details"; press article, section 4):
//   dS_c = phi(K_c)^T diag(eta_c) V_c,   S_c = W1 + sum_{j<c} dS_j (apply-then-update; j <= c for
//   update-then-apply),   O_c = phi(Q_c) S_c.
// One launch, one workgroup per (pair, group of G consecutive chunks); a group behaves as one
// chunk of G*chunk tokens for the scan (its aggregate sums all its tokens; the partial sums at its
// chunk boundaries are kept too) while each chunk's queries still read their own state:
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
// which miss in the per-CU L1. Work lists: list x holds the (pair, group) items of the pairs
// p = x (mod 8) in pair-then-group order; a workgroup takes a ticket from the counter of its XCD
// (hardware XCC id) and works on that item of list x, so a pair's groups share one L2 (the L2s of
// different XCDs are not coherent with each other for these accesses). This needs a device of 8
// XCDs that dispatches the workgroups of a launch to the XCDs in turn (grid / 8 per XCD); the host
// takes this path only on such a device. Forward progress: every predecessor a workgroup may wait
// for holds a smaller ticket of the same list, i.e. has started. Waits are bounded; a timeout
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
  float* agg;               // [pair][nch][rh*h] per group of G chunks: its partial sums at each chunk end,
                            // the last one the group's aggregate (workspace)
  float* incl;              // [pair][nch][rh*h] inclusive prefixes (workspace)
  float* inclm;             // [pair][nch][rh*h] momentum at each inclusive prefix (with momentum)
  float alpha;              // heavy-ball coefficient per chunk (with momentum)
  unsigned* flags;          // [pair][nch]: 1 aggregate published, 2 inclusive prefix published
  unsigned* tickets;        // [8] per-XCD work counters, then the error word at [8]
  int P, heads, N, chunk, nch, inclusive;
  int group;                // chunks per workgroup G (nch % G == 0; G > 1 needs chunk % (NW*32) == 0)
  int64_t w_batch_stride;
  unsigned stress;          // lookback stress (a test hook): nonzero seeds a random delay before
                            // every flag publication, so the lookback meets other orders
};

constexpr long FUSED_SPIN_LIMIT = 1l << 20;

// Lookback stress: a delay of 0 .. 127 sleeps of about a microsecond, from a hash of the seed
// and the publishing (pair, group). Results do not depend on it (the lookback sums in a fixed
// order); only the order in which groups publish changes.
__device__ __forceinline__ void stress_delay(unsigned seed, unsigned key) {
  if (!seed) return;
  unsigned x = key * 2654435761u ^ seed;
  x ^= x >> 15;
  x *= 0x2c1b3c6du;
  x ^= x >> 12;
  for (unsigned k = 0; k < (x & 127u); ++k) __builtin_amdgcn_s_sleep(32);
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

// ID: the identity feature map (RH == H): no fast-weight rows, no token-half combine, and S kept
// transposed ([h][LDT], row reads) for phase C.
template <class OpT, int H, int RH, bool ID = false>
struct FusedLayout {
  static constexpr int NJB = RH / 32, NW = 2 * NJB, NT = 64 * NW;
  static constexpr int LDK = H + Pad<OpT>::v;       // token tiles (row reads and transpose reads)
  static constexpr int LDW = H + Pad<OpT>::v;       // W0^T / W2^T rows
  static constexpr int LD1 = ID ? H + Pad<OpT>::v : tr_ld<OpT>(H);  // S rows (transpose reads), S^T rows (ID)
  static constexpr int TILE = TT * LDK;             // elements of one staged token tile
  static constexpr int NB = 3;                                               // token-tile buffers
  static constexpr int TILES_B = NB * 2 * TILE * (int)sizeof(OpT);           // NB x (K, eta*V)
  static constexpr int OST_B = NW * 32 * (H + 8) * 2;                         // output staging
  static constexpr int R0 = TILES_B > OST_B ? TILES_B : OST_B;
  static constexpr int COMB_O = R0;                                          // token-half combine
  static constexpr int WT_O = COMB_O + (ID ? 0 : NJB * 32 * H * 4);          // W0^T, W2^T [RH][LDW]
  static constexpr int SS_O = WT_O + (ID ? 0 : 2 * RH * LDW * (int)sizeof(OpT));  // S [RH][LD1]
  static constexpr int bytes = SS_O + RH * LD1 * (int)sizeof(OpT) + 16;
  // state float4 groups per thread, aggregates loaded together in the lookback, and the largest
  // group of chunks the momentum lookback holds in registers
  static constexpr int SPT = (RH * H / 4 + NT - 1) / NT;
  static constexpr int LB = SPT >= 8 ? 2 : 8;
  static constexpr int GMAX = SPT >= 8 ? 1 : 8;
};

template <class OpT, int H, int RH, bool ID = false>
constexpr int linattn_fused_lds_bytes() { return FusedLayout<OpT, H, RH, ID>::bytes; }

// grid: 8 * ceil(P / 8) * (nch / G) workgroups; block NT = 128 * RH / 32 threads.
// MOM: heavy-ball momentum per chunk. The carried state is then the pair (S, m): a group of G
// chunks with partial sums P_0..P_{G-1} maps it to (S + A_S + sigma_G m, alpha^G m + A_m), with
// A_S = sum_j alpha^(G-1-j) P_j, A_m = sum_j alpha^(G-1-j) (P_j - P_{j-1}) and
// sigma_L = alpha + ... + alpha^L; the state after L of the group's chunks is
// S + sigma_L m + sum_{j<L} alpha^(L-1-j) P_j. Readers rebuild these sums from the stored
// partial sums, so the aggregate phase is the same as without momentum.
// ID: the identity feature map (RH == H): phase A contracts K and eta*V straight from the staged
// tiles (wave (jb, half) owns rows jb*32.. and half of the columns of dS over all 64 tokens of a
// tile), phase C multiplies the query rows by S.
template <class IoT, class OpT, int H, int RH, bool MOM = false, bool ID = false>
__global__ void __launch_bounds__(128 * (RH / 32)) linattn_fused_kernel(FusedArgs a) {
  typedef Mfma<OpT> M;
  typedef typename M::frag frag;
  typedef FusedLayout<OpT, H, RH, ID> L;
  constexpr int NJB = L::NJB, NW = L::NW, NT = L::NT;
  constexpr int LDK = L::LDK, LDW = L::LDW, LD1 = L::LD1, TILE = L::TILE, NB = L::NB;
  constexpr int KS = H / M::KSTEP;          // K steps over h
  constexpr int QS = 32 / M::KSTEP;         // K steps over 32 tokens / 32 hidden units
  constexpr int CB = H / 32;                // 32-column blocks of h
  constexpr int VE = Io<IoT>::VEC;          // I/O elements per 16-byte chunk
  constexpr int NCK = TT * H / VE;          // 16-byte chunks of one token tile
  constexpr int CPT = (NCK + NT - 1) / NT;
  constexpr int NS4 = RH * H / 4;           // float4 groups of the state
  constexpr int SPT = L::SPT, LB = L::LB, GMAX = L::GMAX;
  constexpr int CBH = CB / 2;               // ID: 32-column blocks of dS per wave
  static_assert(RH % 32 == 0 && H % 32 == 0 && NT <= 1024, "shape");
  static_assert(!ID || (RH == H && H % 64 == 0), "identity map: h x h state, h a multiple of 64");
  static_assert(std::is_same<IoT, bf16_t>::value && std::is_same<OpT, _Float16>::value, "bf16 I/O, fp16 operands");

  extern __shared__ __align__(16) unsigned char smem[];
  OpT* tiles = reinterpret_cast<OpT*>(smem);                       // [NB][K, eta*V][TT][LDK]
  float* comb = reinterpret_cast<float*>(smem + L::COMB_O);        // phase A token-half combine
  bf16_t* ost = reinterpret_cast<bf16_t*>(smem);                   // phase C output staging
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

  // ---- token-tile staging of K and eta*V: NPF register sets rotate, so a tile is requested NPF
  // tiles before it is stored to LDS. Buffer loads over the group's rows return zero past its end,
  // so the staging has no branches. ----
  struct Staged {
    u32x4 k[CPT], v[CPT];
    float e[CPT];
  };
  constexpr int NPF = 2;  // measured at the scan workload: as fast as 3 or 4 sets, fewer registers
  Staged sg4[NPF];
  const int gbytes = (cend - cbase) * H * (int)sizeof(IoT);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<IoT*>(Kp + (int64_t)cbase * H), (short)0, gbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<IoT*>(Vp + (int64_t)cbase * H), (short)0, gbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ep + cbase), (short)0, (cend - cbase) * 4, 0x00020000);
  auto fetch = [&](int tile, Staged& sg) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c16 = tid + NT * i;
      const int row = tile * TT + c16 / (H / VE), col = (c16 % (H / VE)) * VE;
      const int off = (row * H + col) * (int)sizeof(IoT);
      sg.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      sg.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
      sg.e[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, row * 4, 0, 0));
    }
  };
  auto put = [&](int buf, const Staged& sg) {
    OpT* kb = tiles + buf * 2 * TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c16 = tid + NT * i;
      if (NCK % NT == 0 || c16 < NCK) {
        const int row = c16 / (H / VE), col = (c16 % (H / VE)) * VE;
        *reinterpret_cast<f16x8*>(kb + row * LDK + col) = bf16x8_to_f16x8(sg.k[i]);
        *reinterpret_cast<f16x8*>(kb + TILE + row * LDK + col) = bf16x8_scaled_f16x8(sg.v[i], sg.e[i]);
      }
    }
  };

  const int ntile = (G * a.chunk + TT - 1) / TT;
#pragma unroll
  for (int k = 0; k < NPF; ++k) fetch(k, sg4[k]);

  // ---- fast-weight fragments of hidden rows jb*32 + (lane & 31): MFMA B operands in phase A,
  // A operands in phase C (same lane layout); W0^T / W2^T also go to LDS for phase C. W0 is
  // scaled by -log2(e) and W2 by -ln(2): with u = x W0 (-log2 e) and v = x W2 (-ln 2),
  // silu(x W0) (x W2) = u v / (1 + 2^u). ----
  const int jb = w % NJB, th = w / NJB;  // ID: th is the wave's column half of dS
  frag wf[2][KS];
  if constexpr (!ID) {
    const int j = jb * 32 + (lane & 31);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* src = m == 0 ? W0p : W2p;
      const float sc = m == 0 ? -1.4426950408889634f : -0.6931471805599453f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k0 = s * M::KSTEP + (lane >> 5) * M::KSUB;
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[m][s][e] = M::from_f32(src[(int64_t)(k0 + e) * RH + j] * sc);
        if (th == 0) *reinterpret_cast<frag*>(Wt + (m * RH + j) * LDW + k0) = wf[m][s];
      }
    }
  }

  // ---- A. chunk aggregate dS = phi(K)^T diag(eta) V. Token tiles rotate through NB = 3 LDS
  // buffers; iteration i stores tile i+2, reads K of tile i+1 and eta*V of tile i, issues the
  // pre-activation products of tile i+1 between the epilogue instructions of tile i (the matrix
  // cores and the vector ALUs work at the same time), then adds tile i into the aggregate. One
  // barrier per tile. ----
  f32x16 acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) zero(acc[c]);
  const OpT* krow = tiles + (th * 32 + (lane & 31)) * LDK + (lane >> 5) * M::KSUB;
  f32x16 pu[2], pv[2];  // pre-activations u, v of the current and the next tile
  auto tile_iter = [&](int i, int bc, Staged& sp, f32x16& uc, f32x16& vc, f32x16& un, f32x16& vn) {
    const int bn = bc == NB - 1 ? 0 : bc + 1, bp = bn == NB - 1 ? 0 : bn + 1;
    put(bp, sp);  // tile i+2 (past the end: unread)
    fetch(i + 2 + NPF, sp);
    frag kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = M::load(krow + bn * 2 * TILE + s * M::KSTEP);
    frag vf[QS][CB];
    const OpT* vh = tiles + bc * 2 * TILE + TILE + th * 32 * LDK;
#pragma unroll
    for (int q = 0; q < QS; ++q)
#pragma unroll
      for (int c = 0; c < CB; ++c) vf[q][c] = acc_kfrag_tr<OpT>(vh + c * 32, LDK, q, lane);
    __builtin_amdgcn_sched_barrier(0);
    frag hf[QS];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float x0 = uc[r], x1 = uc[r + 1];
      const float y0 = x0 * vc[r] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x0));
      const float y1 = x1 * vc[r + 1] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x1));
      const f16x2 h = f32x2_to_f16x2(y0, y1);
      hf[r >> 3][r & 7] = h[0];
      hf[r >> 3][(r & 7) + 1] = h[1];
    }
    zero(un);
    zero(vn);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      un = M::mma(kf[s], wf[0][s], un);
      vn = M::mma(kf[s], wf[1][s], vn);
    }
#pragma unroll
    for (int q = 0; q < QS; ++q)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[c] = M::mma(hf[q], vf[q][c], acc[c]);
    // schedule: the pre-activation products spread over the epilogue, then the contraction
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
    for (int m = 0; m < 2 * KS; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 88 / (2 * KS), 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QS * CB, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  // ID: iteration i stores tile i+2 and contracts tile i: acc[c] += K^T (eta V) over its 64 tokens
  // (both operands transpose-read with the same token permutation)
  auto tile_id = [&](int bc, Staged& sp, int inext) {
    const int bp = bc == 0 ? NB - 1 : bc - 1;  // buffer of tile i+2 (that of tile i-1)
    put(bp, sp);
    fetch(inext, sp);
    const OpT* kt = tiles + bc * 2 * TILE;
    const OpT* vt = kt + TILE;
    frag hf[2][QS], vf[2][QS][CBH];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        hf[t2][q] = acc_kfrag_tr<OpT>(kt + t2 * 32 * LDK + jb * 32, LDK, q, lane);
#pragma unroll
        for (int c = 0; c < CBH; ++c)
          vf[t2][q][c] = acc_kfrag_tr<OpT>(vt + t2 * 32 * LDK + (th * CBH + c) * 32, LDK, q, lane);
      }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int c = 0; c < CBH; ++c) acc[c] = M::mma(hf[t2][q], vf[t2][q][c], acc[c]);
    __syncthreads();
  };
  // The sums run over the whole group. At the end of the group's chunk i, wave (jb, 1) hands its
  // sums to wave (jb, 0), which adds them (in a fixed order) and stores the group's partial sum
  // through chunk i to slot ch*G + i; slot ch*G + G-1 holds the group's aggregate.
  auto combine = [&](int i) {
    if constexpr (ID) {
      float* ag = aggp + ((int64_t)ch * G + i) * n + (int64_t)jb * 32 * H;
#pragma unroll
      for (int c = 0; c < CBH; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) ag[acc_row(r, lane) * H + (th * CBH + c) * 32 + acc_col(lane)] = acc[c][r];
      return;
    }
    if (th == 1) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) comb[((jb * CB + c) * 16 + r) * 64 + lane] = acc[c][r];
    }
    __syncthreads();
    if (th == 0) {
      float* ag = aggp + ((int64_t)ch * G + i) * n + (int64_t)jb * 32 * H;
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ag[acc_row(r, lane) * H + c * 32 + acc_col(lane)] = acc[c][r] + comb[((jb * CB + c) * 16 + r) * 64 + lane];
    }
  };
  put(0, sg4[0]);
  fetch(NPF, sg4[0]);
  put(1, sg4[1]);
  fetch(NPF + 1, sg4[1]);
  __syncthreads();
  if constexpr (!ID) {
    zero(pu[0]);
    zero(pv[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const frag kf = M::load(krow + s * M::KSTEP);
      pu[0] = M::mma(kf, wf[0][s], pu[0]);
      pv[0] = M::mma(kf, wf[1][s], pv[0]);
    }
  }
  const int tpc = a.chunk / TT;  // tiles per chunk (G > 1: whole tiles)
  int bc = 0;                    // buffer of tile i
  // whole blocks of NPF tiles run without branches between the staging loads and their use, so
  // the loads stay in flight across iterations; the remainder follows
  const int nfull = ntile - ntile % NPF;
  int i0 = 0;
  for (; i0 < nfull; i0 += NPF) {
#pragma unroll
    for (int k = 0; k < NPF; ++k) {
      const int i = i0 + k;
      if constexpr (ID)
        tile_id(bc, sg4[(k + 2) % NPF], i + 2 + NPF);
      else
        tile_iter(i, bc, sg4[(k + 2) % NPF], pu[k & 1], pv[k & 1], pu[(k + 1) & 1], pv[(k + 1) & 1]);
      bc = bc == NB - 1 ? 0 : bc + 1;
      if (G > 1 && (i + 1) % tpc == 0 && i + 1 < ntile) combine(i / tpc);
    }
  }
#pragma unroll
  for (int k = 0; k < NPF - 1; ++k) {
    const int i = i0 + k;
    if (i < ntile) {
      if constexpr (ID)
        tile_id(bc, sg4[(k + 2) % NPF], i + 2 + NPF);
      else
        tile_iter(i, bc, sg4[(k + 2) % NPF], pu[k & 1], pv[k & 1], pu[(k + 1) & 1], pv[(k + 1) & 1]);
      bc = bc == NB - 1 ? 0 : bc + 1;
    }
  }
  combine(G - 1);
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    stress_delay(a.stress, (unsigned)(pair * a.nch + ch) * 2u);
    __hip_atomic_store(fl + ch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // the first query pass's rows are requested now and arrive during the lookback
  u32x4 qa[KS], qb[KS];
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<IoT*>(Qp + (int64_t)cbase * H), (short)0, gbytes, 0x00020000);
  auto load_q = [&](int t0, u32x4 (&qr)[KS]) {  // rows past the group's end read zero
    const int t = t0 - cbase + 32 * w + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = s * M::KSTEP + (lane >> 5) * M::KSUB;
      qr[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (t * H + c) * (int)sizeof(IoT), 0, 0));
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
  f32x4 run[SPT];                // state before the group
  f32x4 mrun[MOM ? SPT : 1];     // momentum before the group
  const float al = a.alpha;
  if constexpr (MOM) {
    // (S, m) = the inclusive prefix at `stop` (or (W1, 0)), then the groups stop+1 .. ch in
    // order, each through its affine map rebuilt from its G partial sums (loaded together)
    const __amdgpu_buffer_rsrc_t rim = dev_rsrc(a.inclm + (int64_t)pair * a.nch * n, (int)(a.nch * n * 4));
    float aG = 1.f, sG = 0.f;
    for (int k = 0; k < G; ++k) {
      aG *= al;
      sG += aG;
    }
    f32x4 s[SPT], m[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      s[i] = stop >= 0 ? dev_load4(ri, (int)((stop * n + e) * 4)) : *reinterpret_cast<const f32x4*>(W1p + e);
      m[i] = stop >= 0 ? dev_load4(rim, (int)((stop * n + e) * 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int g = stop + 1; g <= ch; ++g) {
      f32x4 pj[GMAX][SPT];
#pragma unroll
      for (int j = 0; j < GMAX; ++j)
#pragma unroll
        for (int i = 0; i < SPT; ++i)
          pj[j][i] = j < G ? dev_load4(ra, (int)(((g * G + j) * n + 4 * (tid + NT * i)) * 4))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 aw[SPT], am[SPT];
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        aw[i] = pj[0][i];
        am[i] = pj[0][i];
      }
#pragma unroll
      for (int j = 1; j < GMAX; ++j)
        if (j < G)
#pragma unroll
          for (int i = 0; i < SPT; ++i) {
            aw[i] = al * aw[i] + pj[j][i];
            am[i] = al * am[i] + (pj[j][i] - pj[j - 1][i]);
          }
      if (g == ch)
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
          run[i] = s[i];
          mrun[i] = m[i];
        }
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        s[i] = s[i] + aw[i] + sG * m[i];
        m[i] = aG * m[i] + am[i];
      }
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      *reinterpret_cast<f32x4*>(inclp + (int64_t)ch * n + e) = s[i];
      *reinterpret_cast<f32x4*>(a.inclm + ((int64_t)pair * a.nch + ch) * n + e) = m[i];
      if (ch == ngr - 1 && a.S_out) *reinterpret_cast<f32x4*>(a.S_out + (int64_t)pair * n + e) = s[i];
    }
  } else {
    // prefix = (inclusive prefix at `stop`, or W1) + aggregates stop+1 .. ch-1, left to right;
    // loads of eight aggregates are in flight together
    f32x4 s[SPT], own[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) own[i] = dev_load4(ra, (int)(((ch * G + G - 1) * n + 4 * (tid + NT * i)) * 4));
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      s[i] = stop >= 0 ? dev_load4(ri, (int)((stop * n + e) * 4)) : *reinterpret_cast<const f32x4*>(W1p + e);
    }
    for (int j0 = stop + 1; j0 < ch; j0 += LB) {
      f32x4 t[LB][SPT];
#pragma unroll
      for (int jj = 0; jj < LB; ++jj)
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
          const int e = 4 * (tid + NT * i);
          t[jj][i] = (j0 + jj < ch) ? dev_load4(ra, (int)((((j0 + jj) * G + G - 1) * n + e) * 4))
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int jj = 0; jj < LB; ++jj)
        if (j0 + jj < ch)
#pragma unroll
          for (int i = 0; i < SPT; ++i) s[i] += t[jj][i];
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int e = 4 * (tid + NT * i);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      const f32x4 inc = s[i] + own[i];
      *reinterpret_cast<f32x4*>(inclp + (int64_t)ch * n + e) = inc;
      if (ch == ngr - 1 && a.S_out) *reinterpret_cast<f32x4*>(a.S_out + (int64_t)pair * n + e) = inc;
      run[i] = s[i];
    }
  }
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    stress_delay(a.stress, (unsigned)(pair * a.nch + ch) * 2u + 1u);
    __hip_atomic_store(fl + ch, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- C. O = phi(Q) S for the chunk's query tokens, wave w: 32 tokens per pass, the fast
  // weights and S read from LDS. The hidden blocks are pipelined: the pre-activation products of
  // block j2+1 are issued between the epilogue instructions of block j2. ----
  IoT* Op = reinterpret_cast<IoT*>(a.O) + (int64_t)pair * a.N * H;
  int ocur = cbase;  // first row of the chunk whose outputs are written
  __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(Op + (int64_t)cbase * H, (short)0, a.chunk * H * (int)sizeof(IoT), 0x00020000);
  auto wload = [&](int j2, frag (&a0)[KS], frag (&a2)[KS]) {
    const OpT* r0 = Wt + (j2 * 32 + (lane & 31)) * LDW + (lane >> 5) * M::KSUB;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      a0[s] = M::load(r0 + s * M::KSTEP);
      a2[s] = M::load(r0 + RH * LDW + s * M::KSTEP);
    }
  };
  auto pass = [&](int t0, const u32x4 (&qcur)[KS], u32x4 (&qnext)[KS]) {
    load_q(t0 + NW * 32, qnext);
    const int tw = t0 + 32 * w;
    {
      frag qf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = bf16x8_to_f16x8(qcur[s]);
      // stage the wave's 32 x h output tile in LDS (each lane holds four consecutive columns of a
      // token row), then write whole 16-byte row runs; rows past the chunk end fall outside the
      // store range and are dropped
      bf16_t* os = ost + w * 32 * (H + 8) + (lane & 31) * (H + 8) + 4 * (lane >> 5);
      auto stage = [&](int c, const f32x16& oc) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = f32x2_to_bf16x2_bits(oc[4 * g], oc[4 * g + 1]);
          const uint32_t hi = f32x2_to_bf16x2_bits(oc[4 * g + 2], oc[4 * g + 3]);
          *reinterpret_cast<u32x2*>(os + c * 32 + 8 * g) = u32x2{lo, hi};
        }
      };
      if constexpr (ID) {
        // O^T = S^T Q^T one 32-column block at a time: S^T rows from LDS, the query rows as the
        // B operand
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          f32x16 oc;
          zero(oc);
#pragma unroll
          for (int s = 0; s < KS; ++s)
            oc = M::mma(M::load(Ss + (c * 32 + (lane & 31)) * LD1 + s * M::KSTEP + (lane >> 5) * M::KSUB), qf[s], oc);
          stage(c, oc);
        }
      } else {
      f32x16 o[CB];  // O^T: rows are output columns c*32.., columns the wave's 32 tokens
#pragma unroll
      for (int c = 0; c < CB; ++c) zero(o[c]);
      f32x16 pu[2], pv[2];
      {
        frag a0[KS], a2[KS];
        wload(0, a0, a2);
        zero(pu[0]);
        zero(pv[0]);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          pu[0] = M::mma(a0[s], qf[s], pu[0]);
          pv[0] = M::mma(a2[s], qf[s], pv[0]);
        }
      }
#pragma unroll
      for (int j2 = 0; j2 < NJB; ++j2) {
        f32x16& uc = pu[j2 & 1];
        f32x16& vc = pv[j2 & 1];
        f32x16& un = pu[(j2 + 1) & 1];
        f32x16& vn = pv[(j2 + 1) & 1];
        const bool nx = j2 + 1 < NJB;
        frag a0[KS], a2[KS];
        if (nx) wload(j2 + 1, a0, a2);
        frag sf[QS][CB];
        const OpT* sr = Ss + j2 * 32 * LD1;
#pragma unroll
        for (int q = 0; q < QS; ++q)
#pragma unroll
          for (int c = 0; c < CB; ++c) sf[q][c] = acc_kfrag_tr<OpT>(sr + c * 32, LD1, q, lane);
        __builtin_amdgcn_sched_barrier(0);
        frag hf[QS];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = uc[r], x1 = uc[r + 1];
          const float y0 = x0 * vc[r] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x0));
          const float y1 = x1 * vc[r + 1] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x1));
          const f16x2 h = f32x2_to_f16x2(y0, y1);
          hf[r >> 3][r & 7] = h[0];
          hf[r >> 3][(r & 7) + 1] = h[1];
        }
        if (nx) {
          zero(un);
          zero(vn);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            un = M::mma(a0[s], qf[s], un);
            vn = M::mma(a2[s], qf[s], vn);
          }
        }
#pragma unroll
        for (int q = 0; q < QS; ++q)
#pragma unroll
          for (int c = 0; c < CB; ++c) o[c] = M::mma(sf[q][c], hf[q], o[c]);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        if (nx) {
#pragma unroll
          for (int m = 0; m < 2 * KS; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 88 / (2 * KS), 0);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, QS * CB, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) stage(c, o[c]);
      }
      const bf16_t* ow = ost + w * 32 * (H + 8);
#pragma unroll
      for (int i = lane; i < 32 * H / 8; i += 64) {
        const int row = i / (H / 8), col = (i % (H / 8)) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ow + row * (H + 8) + col);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, ((tw - ocur + row) * H + col) * (int)sizeof(IoT), 0, 0);
      }
    }
  };
  // chunk i of the group reads S = run + the group's partial sum through chunk i-1 (through chunk i
  // when inclusive; the last chunk's inclusive state is then the group's inclusive prefix)
  int np = 0;  // passes so far: even passes read qa and prefetch into qb, odd ones the reverse
  for (int i = 0; i < (MOM && GMAX == 1 ? 1 : G); ++i) {  // (the host keeps G <= GMAX with momentum)
    const int slot = i - (a.inclusive ? 0 : 1);  // group partial sum through chunk `slot`
    f32x4 part[SPT];
    float sL = 0.f;  // with momentum: sigma_L for the L = slot + 1 chunk writes before this state
    if constexpr (MOM) {
      // part = sum_{j<=slot} alpha^(slot-j) P_j (Horner over the group's partial sums)
#pragma unroll
      for (int k = 0; k < SPT; ++k) part[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      float pw = 1.f;
      for (int j = 0; j <= slot; ++j) {
        f32x4 pj[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) pj[k] = dev_load4(ra, (int)(((ch * G + j) * n + 4 * (tid + NT * k)) * 4));
#pragma unroll
        for (int k = 0; k < SPT; ++k) part[k] = al * part[k] + pj[k];
        pw *= al;
        sL += pw;
      }
    } else {
#pragma unroll
      for (int k = 0; k < SPT; ++k) part[k] = dev_load4(ra, (int)(((ch * G + (slot < 0 ? 0 : slot)) * n + 4 * (tid + NT * k)) * 4));
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int e = 4 * (tid + NT * k);
      if (NS4 % NT != 0 && e >= 4 * NS4) continue;
      f32x4 sc = slot < 0 ? run[k] : run[k] + part[k];
      if constexpr (MOM) sc = run[k] + sL * mrun[MOM ? k : 0] + part[k];
      if (bad) sc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      const int j = e / H, c = e % H;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (ID)
          Ss[(c + q) * LD1 + j] = M::from_f32(sc[q]);
        else
          Ss[j * LD1 + c + q] = M::from_f32(sc[q]);
      }
    }
    __syncthreads();  // S of chunk i in LDS
    ocur = cbase + i * a.chunk;
    ro = __builtin_amdgcn_make_buffer_rsrc(Op + (int64_t)ocur * H, (short)0, a.chunk * H * (int)sizeof(IoT), 0x00020000);
    for (int t0 = ocur; t0 < ocur + a.chunk; t0 += NW * 32, ++np) {
      if (np & 1)
        pass(t0, qb, qa);
      else
        pass(t0, qa, qb);
    }
    __syncthreads();  // every wave is done with S before the next chunk's is stored
  }
}

}  // namespace ttt
