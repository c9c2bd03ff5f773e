// Device-side building blocks shared by the linear-attention kernels (gfx950).
//
// Matrix-core conventions used throughout (wave64, MFMA 16x16 output tiles):
//   A operand (16 x K):  lane l supplies row  i = l % 16 and 8 values along k.
//   B operand (K x 16):  lane l supplies col  j = l % 16 and 8 values along k.
//   C/D (16 x 16, fp32): lane l holds rows 4*(l/16) + r, r = 0..3, of col l % 16.
// Lanes of the same group g = l / 16 contribute the same 8 k-indices to A and
// B, so any assignment of k-indices to (g, element) works as long as A and B
// use the same one.  Two assignments appear below:
//   "contiguous": group g takes k = 8g .. 8g+7 of the 32-wide block;
//   "split"     : group g takes k = 4g .. 4g+3 and 16+4g .. 16+4g+3, which is
//                 exactly what a lane holds of two vertically stacked 16x16
//                 accumulator tiles; it lets an accumulator be fed back as an
//                 operand without moving data between lanes.
// bf16 tiles use v_mfma_f32_16x16x32_bf16 (one instruction per 32-wide k
// block); fp32 tiles use eight v_mfma_f32_16x16x4_f32, step e pairing element
// e of every lane group, which covers the same 32 k-indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (the conversion gfx950 performs in hardware).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return static_cast<bf16>(x);
}

// Value of x after rounding to the storage type T (identity for fp32).
template <typename T> __device__ __forceinline__ float round_to(float x) {
  return to_f32(from_f32<T>(x));
}

// ---------------------------------------------------------------------------
// 16-byte vectors: 8 bf16 or 4 fp32 elements.
// ---------------------------------------------------------------------------
// Native 16-byte vector (kept in registers; HIP's uint4 struct can end up in
// scratch memory when copied as a whole).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  union { u32x4 raw; bf16 e[8]; };
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  union { u32x4 raw; float e[4]; };
};

// ---------------------------------------------------------------------------
// MFMA fragments: 8 values of one lane along k.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ f32x4 mma(const Frag<bf16> &a, const Frag<bf16> &b,
                                     f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b,
                                     f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// Contiguous k-assignment: 8 consecutive elements at p (16-byte aligned for
// bf16, 32-byte span for fp32).
__device__ __forceinline__ void load_frag8(Frag<bf16> &f, const bf16 *p) {
  f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag8(Frag<float> &f, const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// Split k-assignment: 4 elements at p0 then 4 at p1.
__device__ __forceinline__ void load_frag44(Frag<bf16> &f, const bf16 *p0,
                                            const bf16 *p1) {
  const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void load_frag44(Frag<float> &f, const float *p0,
                                            const float *p1) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p1);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// ---------------------------------------------------------------------------
// Fragments of a row-major [k][n] tile in LDS whose contraction index k runs
// along rows: lane (g = l / 16, i = l % 16) receives column n0 + i at 8 rows.
//   contiguous assignment: rows k0 + 8g + e, e = 0..7
//   split assignment     : rows k0 + 4g + e and k0 + 16 + 4g + e, e = 0..3
// bf16: gfx950's transposing LDS read (ds_read_b64_tr_b16).  Within each
// 16-lane block, source lane j supplies 4 consecutive 16-bit values and output
// lane i receives value i % 4 of source lanes i/4 + 4e (e = 0..3).  Pointing
// source lane j at row r0 + j/4, columns n0 + 4 (j % 4) therefore hands output
// lane i the 4 values of column n0 + i at rows r0 .. r0 + 3.
// fp32: one 4-byte read per value (16 lanes read 16 consecutive columns).
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 ds_read_tr4(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(const_cast<bf16 *>(p)));
}

// 4 rows r0..r0+3 of column n0 + i (bf16), as elements e0..e0+3 of f.  The
// whole 64-bit result is reinterpreted at once (per-element bit casts of the
// returned vector are not reliable with this compiler).
__device__ __forceinline__ void tr_rows4(Frag<bf16> &f, int e0, const bf16 *base,
                                         int ld, int r0, int n0, int i) {
  const s16x4 v = ds_read_tr4(base + (r0 + i / 4) * ld + n0 + 4 * (i % 4));
  const bf16x4 b = __builtin_bit_cast(bf16x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[e0 + e] = b[e];
}
__device__ __forceinline__ void tr_rows4(Frag<float> &f, int e0, const float *base,
                                         int ld, int r0, int n0, int i) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[e0 + e] = base[(r0 + e) * ld + n0 + i];
}

template <typename T>
__device__ __forceinline__ void load_frag_tr8(Frag<T> &f, const T *base, int ld,
                                              int k0, int n0, int g, int i) {
  tr_rows4(f, 0, base, ld, k0 + 8 * g, n0, i);
  tr_rows4(f, 4, base, ld, k0 + 8 * g + 4, n0, i);
}

template <typename T>
__device__ __forceinline__ void load_frag_tr44(Frag<T> &f, const T *base, int ld,
                                               int k0, int n0, int g, int i) {
  tr_rows4(f, 0, base, ld, k0 + 4 * g, n0, i);
  tr_rows4(f, 4, base, ld, k0 + 16 + 4 * g, n0, i);
}

// ---------------------------------------------------------------------------
// Packed bf16 pairs: one 32-bit word holds elements 2i (low half) and 2i+1.
// ---------------------------------------------------------------------------
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest even and packed (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
// The two bf16 halves of a packed word, widened exactly.
__device__ __forceinline__ float bf16_lo(unsigned u) {
  return __builtin_bit_cast(float, u << 16);
}
__device__ __forceinline__ float bf16_hi(unsigned u) {
  return __builtin_bit_cast(float, u & 0xffff0000u);
}

// Element e of f times the weight of its position: w0 for elements 0..3,
// w1 for 4..7 (rounded back to the operand type).
__device__ __forceinline__ void frag_scale(Frag<bf16> &f, const f32x4 &w0,
                                           const f32x4 &w1) {
  const u32x4 u = __builtin_bit_cast(u32x4, f.v);
  const u32x4 r = {pack_bf16x2(bf16_lo(u[0]) * w0[0], bf16_hi(u[0]) * w0[1]),
                   pack_bf16x2(bf16_lo(u[1]) * w0[2], bf16_hi(u[1]) * w0[3]),
                   pack_bf16x2(bf16_lo(u[2]) * w1[0], bf16_hi(u[2]) * w1[1]),
                   pack_bf16x2(bf16_lo(u[3]) * w1[2], bf16_hi(u[3]) * w1[3])};
  f.v = __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ void frag_scale(Frag<float> &f, const f32x4 &w0,
                                           const f32x4 &w1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] *= w0[e];
    f.v[4 + e] *= w1[e];
  }
}

// Split-assignment fragment from two stacked accumulator tiles (top: k = 0..15
// of the block, bottom: k = 16..31), rounded to the operand type.
__device__ __forceinline__ void frag_from_acc(Frag<bf16> &f, const f32x4 &top,
                                              const f32x4 &bot) {
  const u32x4 w = {pack_bf16x2(top[0], top[1]), pack_bf16x2(top[2], top[3]),
                   pack_bf16x2(bot[0], bot[1]), pack_bf16x2(bot[2], bot[3])};
  f.v = __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ void frag_from_acc(Frag<float> &f, const f32x4 &top,
                                              const f32x4 &bot) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f.v[r] = top[r];
    f.v[4 + r] = bot[r];
  }
}

// Zero the elements of a fragment whose bit pattern in m is clear: m holds,
// per pair of elements (2i, 2i+1), 0xffff in the low and/or high half.
__device__ __forceinline__ void frag_mask(Frag<bf16> &f, const u32x4 &m) {
  f.v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f.v) & m);
}
__device__ __forceinline__ void frag_mask(Frag<float> &f, const u32x4 &m) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (((m[e / 2] >> (16 * (e % 2))) & 1u) == 0u) f.v[e] = 0.f;
}

// Store 4 consecutive values (one accumulator column slice) as type T.
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c,
                                      float d) {
  bf16x4 v;
  v[0] = from_f32<bf16>(a); v[1] = from_f32<bf16>(b);
  v[2] = from_f32<bf16>(c); v[3] = from_f32<bf16>(d);
  *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c,
                                      float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4 *>(p) = v;
}

// ---------------------------------------------------------------------------
// Raw buffer accesses.  A resource covers n bytes at p; an access at byte
// offset voffset + soffset at or past n reads zero and writes nothing (the
// hardware range check, soffset included), so chunk loads and stores need
// no clamps, pointer arithmetic or discard addresses per lane.  Word 3
// selects 32-bit data format, as untyped loads and stores require.
// ---------------------------------------------------------------------------
constexpr int kBufferWord3 = 0x00020000;
// An offset past every resource this library builds (stores there are
// dropped).
constexpr unsigned kNoAccess = 0x7ffffff0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p,
                                                            unsigned n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0,
                                           static_cast<int>(n), kBufferWord3);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r,
                                               unsigned off) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r,
                                              unsigned off, float a, float b,
                                              float c, float d, bf16) {
  const u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r,
                                              unsigned off, float a, float b,
                                              float c, float d, float) {
  const f32x4 v = {a, b, c, d};
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off,
                                         0, 0);
}

// ---------------------------------------------------------------------------
// Feature maps on fp32 values ("Linear attention research 2026" page).
// ---------------------------------------------------------------------------
// elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float elu_plus_one(float x) {
  return x > 0.f ? x + 1.f : expf(x);
}

// The same map with exp(x) as the hardware 2^(x log2 e) (relative error a
// few 1e-7, far below the bf16 rounding that follows), computed with no
// branch and no select: exp(x) >= 1 + x for every x, so
// elu(x) + 1 = max(x + 1, min(exp(x), 1)), and min(2^y, 1) is the exp
// instruction's output clamp to [0, 1].
__device__ __forceinline__ float elu_plus_one_fast(float x) {
  const float e = __builtin_amdgcn_fmed3f(
      __builtin_amdgcn_exp2f(x * 1.4426950408889634f), 0.f, 1.f);
  return fmaxf(x + 1.f, e);
}

// g^k for an integer k >= 0, with g^0 = 1 exactly (also for g = 0).
__device__ __forceinline__ float pow_int(float g, float log2g, int64_t k) {
  return k == 0 ? 1.f : exp2f(static_cast<float>(k) * log2g);
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  // Sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
