// One autoregressive decode step per (sequence, head) unit.
//
// "3.2 Reducing d" (efficient1 page), remark after eq 27: keep the two sums
// sum phi(k)^T v and sum phi(k)^T, update them when a new key and value
// arrive, and serve any later query from them.  The update is eqs 7-8 (no
// decay) or eqs 10-11 (decay a) of "2.2 Linear Attention"; the readout is the
// causal form of eq 9, taken from the updated sums:
//   mu' = g mu + b k'^T v,   nu' = g nu + b k',   out = q' mu' / q' . nu'.
//
// The step is bound by HBM: per unit it streams mu (d' x d fp32) in and out
// once.  One 256-thread workgroup per unit; each thread owns one float4 column
// slice of mu and walks d'/rows_per_pass rows of it: all its loads are issued
// before any arithmetic (so each thread keeps d'/rows_per_pass 16-byte loads
// in flight), then it updates, stores, and accumulates q'_f mu'[f][j..j+3].
// The column partials are reduced through LDS in a fixed order (bitwise
// deterministic), and q'.nu' by a fixed-order wave/LDS tree.
//
// Gated form (ROWS): every state row f decays by its own gamma_f =
// exp(lam_f) with input weight 1 - gamma_f, lam given per row and head
// (the diagonal A of "2.3 State-Space Models" eqs 21-25), per unit (the
// input-dependent decay of Mamba's selective step, "Linear attention
// research 2026" page), or per unit and row.
#include "la_device.h"
#include "la_internal.h"

namespace la {

namespace {

constexpr int kDecThreads = 256;

template <typename T>
__device__ __forceinline__ float load_f32(const T *p) { return to_f32(*p); }

// Deterministic block sum of one value per thread; result in every thread.
__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kDecThreads / kWave; ++i) s += red[i];
  return s;
}

// Layouts of the gated decode's log decay (la_decay_layout).
constexpr int kLdChannel = 0, kLdPosition = 1, kLdBoth = 2;

template <typename T, int D, int DF, bool ROWS>
__global__ __launch_bounds__(kDecThreads) void la_decode_kernel(
    float *__restrict__ mu, float *__restrict__ nu, const T *__restrict__ q,
    const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ out,
    int H, int map, const float *__restrict__ omega,
    const float *__restrict__ decay, int ld_layout) {
  constexpr int TPR = D / 4;                 // threads per mu row (float4)
  constexpr int RPP = kDecThreads / TPR;     // rows per pass
  constexpr int ITER = (DF + RPP - 1) / RPP;
  __shared__ float qf[DF], kf[DF], vv[D], xq[D], xk[D];
  __shared__ float red[RPP][D];
  __shared__ float red4[kDecThreads / kWave];
  // gated form: decay and input weight of every row
  __shared__ float grow[ROWS ? DF : 1], brow[ROWS ? DF : 1];

  const int tid = threadIdx.x;
  const int64_t u = blockIdx.x;
  const int h = static_cast<int>(u % H);
  const float g = !ROWS && decay ? decay[h] : 1.f;
  const float b = !ROWS && decay ? 1.f - g : 1.f;
  if constexpr (ROWS) {
    // decay holds log gamma in the given layout
    for (int f = tid; f < DF; f += kDecThreads) {
      const float lam = ld_layout == kLdChannel ? decay[h * DF + f]
                        : ld_layout == kLdPosition ? decay[u]
                                                   : decay[u * DF + f];
      grow[f] = expf(lam);
      brow[f] = -expm1f(lam);  // 1 - gamma, accurate for gamma near 1
    }
  }

  // ---- features of the new token ----
  if (map == 2) {
    // Performer: phi_r = exp(x . omega[:, r] - |x|^2/2) / sqrt(m), m = DF.
    for (int c = tid; c < D; c += kDecThreads) {
      xq[c] = load_f32(q + u * D + c);
      xk[c] = load_f32(k + u * D + c);
    }
    __syncthreads();
    float pq = 0.f, pk = 0.f;
    for (int c = tid; c < D; c += kDecThreads) {
      pq += xq[c] * xq[c];
      pk += xk[c] * xk[c];
    }
    const float hq = 0.5f * block_sum(pq, red4);
    const float hk = 0.5f * block_sum(pk, red4);
    const float inv_sqrt_m = 1.f / sqrtf(static_cast<float>(DF));
    for (int r = tid; r < DF; r += kDecThreads) {
      float uq = 0.f, uk = 0.f;
      for (int c = 0; c < D; ++c) {
        const float om = omega[c * DF + r];
        uq += xq[c] * om;
        uk += xk[c] * om;
      }
      qf[r] = expf(uq - hq) * inv_sqrt_m;
      kf[r] = expf(uk - hk) * inv_sqrt_m;
    }
  } else {
    for (int f = tid; f < DF; f += kDecThreads) {
      const float xq0 = load_f32(q + u * DF + f), xk0 = load_f32(k + u * DF + f);
      qf[f] = map == 1 ? elu_plus_one(xq0) : xq0;
      kf[f] = map == 1 ? elu_plus_one(xk0) : xk0;
    }
  }
  for (int j = tid; j < D; j += kDecThreads) vv[j] = load_f32(v + u * D + j);
  __syncthreads();

  // ---- nu' = g nu + b k' and the denominator q' . nu' ----
  float part = 0.f;
  for (int f = tid; f < DF; f += kDecThreads) {
    const float gf = ROWS ? grow[f] : g, bf = ROWS ? brow[f] : b;
    const float nn = gf * nu[u * DF + f] + bf * kf[f];
    nu[u * DF + f] = nn;
    part += qf[f] * nn;
  }
  const float den = block_sum(part, red4);

  // ---- stream mu: load all, update, store, accumulate q'_f mu'[f][:] ----
  const int j4 = tid % TPR, f0 = tid / TPR;
  float *mub = mu + u * static_cast<int64_t>(DF) * D + 4 * j4;
  f32x4 m[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int f = f0 + RPP * i;
    if (f < DF) m[i] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4 *>(mub + f * D));
  }
  const f32x4 v4 = {vv[4 * j4], vv[4 * j4 + 1], vv[4 * j4 + 2], vv[4 * j4 + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int f = f0 + RPP * i;
    if (f < DF) {
      const float gf = ROWS ? grow[f] : g, bf = ROWS ? brow[f] : b;
      const f32x4 nm = gf * m[i] + (bf * kf[f]) * v4;
      __builtin_nontemporal_store(nm, reinterpret_cast<f32x4 *>(mub + f * D));
      acc += qf[f] * nm;
    }
  }
  red[f0][4 * j4] = acc[0];
  red[f0][4 * j4 + 1] = acc[1];
  red[f0][4 * j4 + 2] = acc[2];
  red[f0][4 * j4 + 3] = acc[3];
  __syncthreads();
  for (int j = tid; j < D; j += kDecThreads) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][j];
    out[u * D + j] = from_f32<T>(s / den);
  }
}

// ld_layout < 0: decay is [H] (or null); else decay holds log gamma in that
// layout (the gated form).
template <typename T, int D, int DF>
hipError_t run_decode(float *mu, float *nu, const void *q, const void *k,
                      const void *v, void *out, int64_t units, int H, int map,
                      const float *omega, const float *decay, int ld_layout,
                      hipStream_t s) {
  if (ld_layout >= 0)
    hipLaunchKernelGGL((la_decode_kernel<T, D, DF, true>), dim3(units),
                       dim3(kDecThreads), 0, s, mu, nu,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<T *>(out), H,
                       map, omega, decay, ld_layout);
  else
    hipLaunchKernelGGL((la_decode_kernel<T, D, DF, false>), dim3(units),
                       dim3(kDecThreads), 0, s, mu, nu,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<T *>(out), H,
                       map, omega, decay, ld_layout);
  return hipGetLastError();
}

using DecodeFn = hipError_t (*)(float *, float *, const void *, const void *,
                                const void *, void *, int64_t, int, int,
                                const float *, const float *, int,
                                hipStream_t);

template <typename T, int D>
DecodeFn decode_by_feat(int df) {
  switch (df) {
    case 16: return &run_decode<T, D, 16>;
    case 32: return &run_decode<T, D, 32>;
    case 64: return &run_decode<T, D, 64>;
    case 128: return &run_decode<T, D, 128>;
    case 256: return &run_decode<T, D, 256>;
    default: return nullptr;
  }
}

template <typename T>
DecodeFn decode_fn(int d, int df) {
  switch (d) {
    case 16: return decode_by_feat<T, 16>(df);
    case 32: return decode_by_feat<T, 32>(df);
    case 64: return decode_by_feat<T, 64>(df);
    case 128: return decode_by_feat<T, 128>(df);
    default: return nullptr;
  }
}

}  // namespace

bool decode_supported(int d, int d_feat) {
  return decode_fn<bf16>(d, d_feat) != nullptr;
}

hipError_t launch_decode(float *mu, float *nu, const void *q, const void *k,
                         const void *v, void *out, int64_t units, int H, int d,
                         int d_feat, int map, const float *omega,
                         const float *decay, int dtype, hipStream_t s,
                         int ld_layout) {
  DecodeFn fn = dtype == 1 ? decode_fn<bf16>(d, d_feat)
                           : decode_fn<float>(d, d_feat);
  if (!fn) return hipErrorInvalidValue;
  return fn(mu, nu, q, k, v, out, units, H, map, omega, decay, ld_layout, s);
}

}  // namespace la
