// common.hpp -- shared device helpers for the gfx950 kernels of the TTT fast-weight library.
//
// MFMA conventions used everywhere (CDNA wave64):
//   A wave computes a 32x32 fp32 tile C += A * B^T where A is [32 x K] and B is [32 x K], both
//   K-contiguous ("row of A", "row of B" each hold one output row / column). Lane l supplies
//   row (l & 31) of A and of B, with the K elements [kk + KSUB*(l>>5), +KSUB) of each K step.
//   The accumulator element acc[r] of lane l is C[i][j] with
//     i = 8*(r/4) + 4*(l>>5) + (r&3),   j = l & 31.
//   16-bit operands use v_mfma_f32_32x32x16_{f16,bf16} (K step 16, 8 elements per lane);
//   fp32 operands use v_mfma_f32_32x32x2f32 (K step 2, 1 element per lane).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ttt {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bfloat16 bit pattern stored in memory (I/O dtype TTT_BF16).
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ------------------------------------------------------------------------------------------
// Operand traits: how a K-contiguous operand row is turned into MFMA fragments.
// ------------------------------------------------------------------------------------------
template <class T> struct Mfma;

template <> struct Mfma<_Float16> {
  static constexpr int KSTEP = 16;   // K per instruction
  static constexpr int KSUB = 8;     // K elements per lane per instruction
  typedef f16x8 frag;
  __device__ __forceinline__ static frag load(const _Float16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static _Float16 from_f32(float x) { return static_cast<_Float16>(x); }
};

template <> struct Mfma<__bf16> {
  static constexpr int KSTEP = 16;
  static constexpr int KSUB = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static frag load(const __bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static __bf16 from_f32(float x) { return static_cast<__bf16>(x); }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KSUB = 1;
  typedef float frag;
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};

// C += A[32 x K] * B[32 x K]^T with A, B K-contiguous rows (lda/ldb in elements).
template <class T, int K>
__device__ __forceinline__ void mma_tile(f32x16& acc, const T* a, int lda, const T* b, int ldb,
                                         int lane) {
  typedef Mfma<T> M;
  const T* ap = a + (lane & 31) * lda + (lane >> 5) * M::KSUB;
  const T* bp = b + (lane & 31) * ldb + (lane >> 5) * M::KSUB;
#pragma unroll
  for (int k = 0; k < K; k += M::KSTEP) acc = M::mma(M::load(ap + k), M::load(bp + k), acc);
}

// Runtime-K variant (K a multiple of the K step).
template <class T>
__device__ __forceinline__ void mma_tile_rt(f32x16& acc, const T* a, int lda, const T* b, int ldb,
                                            int K, int lane) {
  typedef Mfma<T> M;
  const T* ap = a + (lane & 31) * lda + (lane >> 5) * M::KSUB;
  const T* bp = b + (lane & 31) * ldb + (lane >> 5) * M::KSUB;
  for (int k = 0; k < K; k += M::KSTEP) acc = M::mma(M::load(ap + k), M::load(bp + k), acc);
}

// Split-bf16 product of fp32 operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi);
// C += A*B^T ~= hi_a hi_b + hi_a lo_b + lo_a hi_b (relative error ~2^-16 per product).
__device__ __forceinline__ void split8(const float* p, bf16x8& hi, bf16x8& lo) {
  f32x4 v0 = *reinterpret_cast<const f32x4*>(p);
  f32x4 v1 = *reinterpret_cast<const f32x4*>(p + 4);
  float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = static_cast<__bf16>(v[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
  }
}

__device__ __forceinline__ void mma_tile_split(f32x16& acc, const float* a, int lda, const float* b,
                                               int ldb, int K, int lane) {
  const float* ap = a + (lane & 31) * lda + (lane >> 5) * 8;
  const float* bp = b + (lane & 31) * ldb + (lane >> 5) * 8;
  for (int k = 0; k < K; k += 16) {
    bf16x8 ah, al, bh, bl;
    split8(ap + k, ah, al);
    split8(bp + k, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
  }
}

// K-major operand fragment from LDS with the gfx950 transpose read (ds_read_b64_tr_b16).
// The tile is row-major with K along rows: element (k, n) at base[k * ld + n] (16-bit type T).
// Lane l receives n = l & 31 and k = k0 + 8*(l >> 5) + 0..7, i.e. the same fragment that
// Mfma<T>::load gives for an n-major tile. Each 16-lane group addresses a 4 x 16 block
// (lane s of the group: row s / 4, 4-element chunk s % 4) and lane i of the group receives
// column i of the block, rows 0..3; two reads cover the 8 k values. `ld` must keep every
// 4-element chunk 8-byte aligned.
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_tr(const T* base, int ld, int k0, int lane) {
  static_assert(sizeof(T) == 2, "16-bit operands");
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  const int g = lane >> 4, s = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (s >> 2);
  const int col = 16 * (g & 1) + 4 * (s & 3);
  const T* p0 = base + row * ld + col;
  const T* p1 = p0 + 4 * ld;
  v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4*)((__attribute__((address_space(3))) T*)(p0)));
  v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4*)((__attribute__((address_space(3))) T*)(p1)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, v);
}

// Operand fragments that continue from an accumulator tile C[t][j] (32 x 32, fp32, lane layout
// above) into a product contracting over t. Element r of lane l holds t = 8*(r/4) + 4*(l>>5) + r%4,
// so with 16-bit operands K step q (q = 0, 1) takes elements r = 8q .. 8q+7 of every lane: lane
// half g then supplies t = 16q + {4g..4g+3, 8+4g..8+4g+3}. The partner operand must present the
// same t permutation: acc_kfrag_tr reads rows of a row-major (t-major) LDS tile accordingly.
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag acc_to_afrag(const f32x16& c, int q) {
  typename Mfma<T>::frag f;
  if constexpr (Mfma<T>::KSUB == 1) {
    f = c[q];  // fp32: one element per K step of 2, step index q = r
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = Mfma<T>::from_f32(c[8 * q + e]);
  }
  return f;
}

// Partner of acc_to_afrag: element (t, n) at base[t * ld + n] with t relative to the
// accumulator tile's first row; lane l receives n = l & 31 and the permuted t set of K step q.
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag acc_kfrag_tr(const T* base, int ld, int q, int lane) {
  if constexpr (Mfma<T>::KSUB == 1) {
    // fp32 K step q = r: lane half g supplies t = 8*(r/4) + 4*g + r%4
    const int t = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
    return base[t * ld + (lane & 31)];
  } else {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    const int g = lane >> 4, s = lane & 15;
    const int row = 16 * q + 4 * (g >> 1) + (s >> 2);
    const int col = 16 * (g & 1) + 4 * (s & 3);
    const T* p0 = base + row * ld + col;
    const T* p1 = p0 + 8 * ld;
    v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)((__attribute__((address_space(3))) T*)(p0)));
    v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)((__attribute__((address_space(3))) T*)(p1)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(typename Mfma<T>::frag, v);
  }
}

// Row / column of accumulator element r for lane l (see the header comment).
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// ------------------------------------------------------------------------------------------
// I/O element loads: 8 consecutive elements of a token row, converted to the operand type.
// ------------------------------------------------------------------------------------------
template <class IoT> struct Io;

// 8 bf16 (one 16-byte chunk) to 8 fp16: each 32-bit word holds two bf16, which become fp32 by
// placing them in the high half; v_cvt_pkrtz then packs the pair. Every bf16 value inside the
// fp16 range has at most 8 significant bits, so the round-toward-zero pack is exact there.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(u32x4 raw) {
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, raw[i] << 16);
    const float hi = __builtin_bit_cast(float, raw[i] & 0xffff0000u);
    o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return __builtin_bit_cast(f16x8, o);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two fp32 values to fp16, round to nearest even (one packed conversion)
__device__ __forceinline__ f16x2 f32x2_to_f16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector((f2){a, b}, f16x2);
}

// two fp32 values to a packed bf16 pair (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}

// 8 bf16 values times s, rounded to fp16 (round to nearest even)
__device__ __forceinline__ f16x8 bf16x8_scaled_f16x8(u32x4 raw, float s) {
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, raw[i] << 16) * s;
    const float hi = __builtin_bit_cast(float, raw[i] & 0xffff0000u) * s;
    const f16x2 h = f32x2_to_f16x2(lo, hi);
    o[2 * i] = h[0];
    o[2 * i + 1] = h[1];
  }
  return o;
}

template <> struct Io<bf16_t> {
  static constexpr int VEC = 8;  // elements per 16-byte load
  template <class T>
  __device__ __forceinline__ static void load_cvt(const bf16_t* p, T* out) {
    if constexpr (std::is_same<T, _Float16>::value) {
      const f16x8 h = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(p));
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = h[e];
    } else {
      u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = Mfma<T>::from_f32(bf16_to_f32(v[e]));
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }
};

template <> struct Io<float> {
  static constexpr int VEC = 4;
  template <class T>
  __device__ __forceinline__ static void load_cvt(const float* p, T* out) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = Mfma<T>::from_f32(v[e]);
  }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};

// Block-wide sum of one float per thread (any blockDim that is a multiple of 64, <= 1024).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
// The XCD (accelerator complex die) this wave runs on (HW_REG_XCC_ID[3:0]).
__device__ __forceinline__ unsigned hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15;
}

// Workgroup barrier that orders LDS accesses only: global memory operations of the waves may
// still be in flight when it releases (__syncthreads would wait for them as well).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline float block_sum(float v, float* red /* >= 16 floats of LDS */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

}  // namespace ttt
