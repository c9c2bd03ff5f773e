// Feature maps phi applied row by row ("Linear attention research 2026" page:
// elu(x) + 1 for the Linear Transformer; exp(x omega - |x|^2/2)/sqrt(m) for
// Performer random features; Q' = phi(Q), K' = phi(K) of "2.2 Linear
// Attention").
//
// Performer: the projection u = x omega is a [rows x d] x [d x m] contraction
// on the bf16 matrix cores.  omega (fp32) is split once per workgroup into a
// bf16 pair hi + lo (hi = rn(omega), lo = rn(omega - hi)) staged transposed in
// LDS; u accumulates x.hi + x.lo in fp32 (plus x_lo.hi for fp32 inputs, x
// split the same way), which keeps u close to an fp32 product while running on
// the bf16 units.  |x|^2 is summed in fp32 from the stored inputs, and
// exp(u - |x|^2/2)/sqrt(m) is applied in the accumulator registers before the
// store.  Each wave computes u^T for 16 rows (A = omega^T from LDS, B = x rows
// straight from global memory), so its accumulator holds 4 consecutive
// features of one row per lane: one 8- or 16-byte store each.
#include "la_device.h"
#include "la_internal.h"

namespace la {

namespace {

constexpr int kFmThreads = 256;

template <typename Tin, typename Tout>
__global__ __launch_bounds__(kFmThreads) void la_featmap_elem_kernel(
    const Tin *__restrict__ x, Tout *__restrict__ y, int64_t n4, int elu1) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFmThreads + threadIdx.x;
       i < n4; i += static_cast<int64_t>(gridDim.x) * kFmThreads) {
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xv = to_f32(x[4 * i + e]);
      f[e] = elu1 ? elu_plus_one(xv) : xv;
    }
    store4(y + 4 * i, f[0], f[1], f[2], f[3]);
  }
}

// 8 consecutive stored elements as fp32 (zeros when !ok).
__device__ __forceinline__ void load8(float *f, const bf16 *p, bool ok) {
  Vec16<bf16> v;
  v.raw = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = to_f32(v.e[e]);
}
__device__ __forceinline__ void load8(float *f, const float *p, bool ok) {
  Vec16<float> a, b;
  a.raw = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0, 0, 0, 0};
  b.raw = ok ? *reinterpret_cast<const u32x4 *>(p + 4) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = a.e[e];
    f[4 + e] = b.e[e];
  }
}

// Split an fp32 value into bf16 hi + lo.
__device__ __forceinline__ void split_bf16(float v, bf16 &hi, bf16 &lo) {
  hi = from_f32<bf16>(v);
  lo = from_f32<bf16>(v - to_f32(hi));
}

template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kFmThreads) void la_featmap_performer_kernel(
    const Tin *__restrict__ x, Tout *__restrict__ y,
    const float *__restrict__ omega, int64_t rows, int m) {
  constexpr int DP = D < 32 ? 32 : D;     // padded contraction width
  constexpr int LW = DP + 8;              // bf16 row stride of omega^T
  constexpr bool XSPLIT = sizeof(Tin) == 4;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16 *sWh = reinterpret_cast<bf16 *>(smem);
  bf16 *sWl = sWh + m * LW;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;

  // omega [D][m] -> omega^T hi/lo [m][DP] (zero padding for D < 32): each
  // thread takes 4 consecutive features of one row of omega per piece, and
  // the loads of 8 pieces are issued before any is written (one round trip
  // to the cache per 8 pieces instead of one per value)
  {
    const int m4 = m / 4, pieces = m4 * DP;
    constexpr int BATCH = 8;
    for (int base = tid; base < pieces; base += kFmThreads * BATCH) {
      f32x4 v[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = base + kFmThreads * j, c = i / m4, r = 4 * (i % m4);
        v[j] = i < pieces && c < D
                   ? *reinterpret_cast<const f32x4 *>(omega + c * m + r)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int i = base + kFmThreads * j, c = i / m4, r = 4 * (i % m4);
        if (i < pieces) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bf16 hi, lo;
            split_bf16(v[j][e], hi, lo);
            sWh[(r + e) * LW + c] = hi;
            sWl[(r + e) * LW + c] = lo;
          }
        }
      }
    }
  }
  __syncthreads();
  const float inv_sqrt_m = 1.f / sqrtf(static_cast<float>(m));

  for (int64_t tile = blockIdx.x; tile * 64 < rows; tile += gridDim.x) {
    const int64_t row = tile * 64 + 16 * w + li;
    const bool valid = row < rows;
    // B operand: x row `row`, contraction index c = 32 kb + 8 g + e.
    Frag<bf16> xh[DP / 32], xl[DP / 32];
    float sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < DP / 32; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      float xv[8];
      load8(xv, x + row * D + c0, valid && c0 < D);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += xv[e] * xv[e];
        bf16 hi, lo;
        split_bf16(xv[e], hi, lo);
        xh[kb].v[e] = hi;
        xl[kb].v[e] = lo;
      }
    }
    sq = wave_sum_groups(sq);
    const float half_sq = 0.5f * sq;
    for (int rb = 0; rb < m / 16; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DP / 32; ++kb) {
        Frag<bf16> wh, wl;
        load_frag8(wh, sWh + (16 * rb + li) * LW + 32 * kb + 8 * g);
        load_frag8(wl, sWl + (16 * rb + li) * LW + 32 * kb + 8 * g);
        acc = mma(wl, xh[kb], acc);
        if (XSPLIT) acc = mma(wh, xl[kb], acc);
        acc = mma(wh, xh[kb], acc);
      }
      // acc[rr] = u[row][r] with r = 16 rb + 4 g + rr
      if (valid)
        store4(y + row * m + 16 * rb + 4 * g,
               expf(acc[0] - half_sq) * inv_sqrt_m,
               expf(acc[1] - half_sq) * inv_sqrt_m,
               expf(acc[2] - half_sq) * inv_sqrt_m,
               expf(acc[3] - half_sq) * inv_sqrt_m);
    }
  }
}

template <typename Tin, typename Tout, int D>
hipError_t run_performer(const void *x, void *y, const float *omega,
                         int64_t rows, int m, hipStream_t s) {
  constexpr int DP = D < 32 ? 32 : D;
  const size_t lds = sizeof(bf16) * 2 * static_cast<size_t>(m) * (DP + 8);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static const hipError_t once = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&la_featmap_performer_kernel<Tin, Tout, D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (once != hipSuccess) return once;
  // one round of resident workgroups (two per compute unit), each filling
  // omega^T once and then taking every grid-th tile
  const int64_t tiles = (rows + 63) / 64;
  const int64_t grid = tiles < 2 * kCUs ? tiles : 2 * kCUs;
  hipLaunchKernelGGL((la_featmap_performer_kernel<Tin, Tout, D>), dim3(grid),
                     dim3(kFmThreads), lds, s, static_cast<const Tin *>(x),
                     static_cast<Tout *>(y), omega, rows, m);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t performer_by_d(const void *x, void *y, const float *omega,
                          int64_t rows, int d, int m, hipStream_t s) {
  switch (d) {
    case 16: return run_performer<Tin, Tout, 16>(x, y, omega, rows, m, s);
    case 32: return run_performer<Tin, Tout, 32>(x, y, omega, rows, m, s);
    case 64: return run_performer<Tin, Tout, 64>(x, y, omega, rows, m, s);
    case 128: return run_performer<Tin, Tout, 128>(x, y, omega, rows, m, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename Tin, typename Tout>
hipError_t run_elem(const void *x, void *y, int64_t count, int elu1,
                    hipStream_t s) {
  const int64_t n4 = count / 4;
  int64_t grid = (n4 + kFmThreads - 1) / kFmThreads;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((la_featmap_elem_kernel<Tin, Tout>), dim3(grid),
                     dim3(kFmThreads), 0, s, static_cast<const Tin *>(x),
                     static_cast<Tout *>(y), n4, elu1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_featmap_elementwise(const void *x, void *y, int64_t count,
                                      int elu1, int in_dt, int out_dt,
                                      hipStream_t s) {
  if (in_dt == 1 && out_dt == 1) return run_elem<bf16, bf16>(x, y, count, elu1, s);
  if (in_dt == 1 && out_dt == 0) return run_elem<bf16, float>(x, y, count, elu1, s);
  if (in_dt == 0 && out_dt == 1) return run_elem<float, bf16>(x, y, count, elu1, s);
  return run_elem<float, float>(x, y, count, elu1, s);
}

hipError_t launch_featmap_performer(const void *x, void *y, const float *omega,
                                    int64_t rows, int d, int m, int in_dt,
                                    int out_dt, hipStream_t s) {
  if (in_dt == 1 && out_dt == 1)
    return performer_by_d<bf16, bf16>(x, y, omega, rows, d, m, s);
  if (in_dt == 1 && out_dt == 0)
    return performer_by_d<bf16, float>(x, y, omega, rows, d, m, s);
  if (in_dt == 0 && out_dt == 1)
    return performer_by_d<float, bf16>(x, y, omega, rows, d, m, s);
  return performer_by_d<float, float>(x, y, omega, rows, d, m, s);
}

namespace {
__global__ __launch_bounds__(256) void la_fill_zero_kernel(float *p,
                                                           int64_t count) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < count; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.f;
}
}  // namespace

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(la_fill_zero_kernel, dim3(grid), dim3(256), 0, stream, p,
                     count);
  return hipGetLastError();
}

}  // namespace la
