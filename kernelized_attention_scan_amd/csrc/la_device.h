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
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  union { uint4 raw; bf16 e[8]; };
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  union { uint4 raw; float e[4]; };
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

// Split-assignment fragment from two stacked accumulator tiles (top: k = 0..15
// of the block, bottom: k = 16..31), rounded to the operand type.
template <typename T>
__device__ __forceinline__ void frag_from_acc(Frag<T> &f, const f32x4 &top,
                                              const f32x4 &bot) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f.v[r] = from_f32<T>(top[r]);
    f.v[4 + r] = from_f32<T>(bot[r]);
  }
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
// Feature maps on fp32 values ("Linear attention research 2026" page).
// ---------------------------------------------------------------------------
// elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float elu_plus_one(float x) {
  return x > 0.f ? x + 1.f : expf(x);
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
