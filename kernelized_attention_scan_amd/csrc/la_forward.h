// Chunked causal kernelized linear attention on gfx950 matrix cores.
//
// The method ("2.2 Linear Attention", efficient2 page, eqs 7-11 and the causal
// form of eq 9) is a per-position recurrence over a d' x d state.  On the GPU
// it is regrouped exactly into chunks of C positions (local index t, s in
// [0, C), state S, z before the chunk, g = a, b = 1 - a with decay, g = b = 1
// without):
//
//   P[t][s]  = b g^(t-s) (q'_t . k'_s) for s <= t, else 0   (masked quadratic
//              form of "3.2 Reducing d" eqs 19-27, efficient1 page)
//   num_t    = sum_s P[t][s] v_s + g^(t+1) q'_t S
//   den_t    = sum_s P[t][s]     + g^(t+1) q'_t . z
//   out_t    = num_t / den_t
//   S       <- g^r S + sum_{s<r} b g^(r-1-s) k'_s^T v_s   (r valid rows)
//   z       <- g^r z + sum_{s<r} b g^(r-1-s) k'_s
//
// Unrolling eqs 10-11 from a state S gives mu_{t} = g^(t+1) S + sum_{s<=t}
// b g^(t-s) k'_s^T v_s, which is what the first three lines read out, and the
// state after the chunk, which is the last two.  With no decay every weight
// is 1 (eqs 7-8).
//
// Sequence parallelism: each (batch, head) unit's sequence is cut into
// segments of whole chunks.  Kernel `agg` computes every segment's aggregate
// (its end state starting from zero); kernel `scan` turns the aggregates into
// exclusive prefixes in place (state entering segment s = g^len * previous +
// aggregate) and appends the total; kernel `fwd` then runs the chunk loop of
// every segment from its prefix.  Non-causal attention (eq 9 with mu_n, nu_n)
// reads the total in every segment.
//
// Work split inside a 256-thread workgroup (4 waves):
//   - staging: all threads load the chunk's Q, K, V with 16-byte coalesced
//     loads (prefetched one chunk ahead in registers), apply phi in fp32 and
//     write the operand tiles to LDS: Q' and K' row-major, (w . K')^T and V^T
//     transposed (w_s = b g^(r-1-s), the state-update weights);
//   - readout: wave w owns 16-row output strips; it forms its strip of P^T on
//     the matrix cores, feeds the accumulator straight back as the B operand
//     of V^T P^T ("split" k-assignment), and adds S^T Q'^T from a bf16 copy of
//     S^T kept in LDS;
//   - state: the fp32 state S lives in registers as 16x16 accumulator tiles
//     spread over the waves; each chunk adds (w.K')^T V on the matrix cores.
#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kMaxLds = 160 * 1024;

template <typename T, int D, int DF>
struct FwdShape {
  // Chunk rows: 64 for bf16 operands; 32 where LDS would not hold 64.
  static constexpr int C =
      (sizeof(T) == 2 && !(DF == 256 && D == 128)) ? 64 : 32;
  static constexpr int DFP = DF < 32 ? 32 : DF;      // padded k-width of q', k'
  static constexpr int PADE = 16 / sizeof(T);        // 16-byte row padding
  static constexpr int LQ = DFP + PADE;              // sQ, sK row stride
  static constexpr int LT = C + PADE;                // sKT, sVT row stride
  static constexpr int LS = DFP + PADE;              // sST row stride
  static constexpr int STRIPS = C / 16;
  static constexpr int NJ = D / 16, NF = DF / 16;
  static constexpr int NTILE = NF * NJ;              // 16x16 state tiles
  static constexpr int TPW = (NTILE + kWaves - 1) / kWaves;
  static constexpr int SQ = C * LQ, SK = C * LQ, SKT = DF * LT, SVT = D * LT,
                       SST = D * LS;
  static constexpr size_t lds_fwd =
      sizeof(T) * (SQ + SK + SKT + SVT + SST) + sizeof(float) * (DF + C + 1);
  static constexpr size_t lds_agg =
      sizeof(T) * (SKT + SVT) + sizeof(float) * (C + 1);
  // fp32 state slot: NTILE tiles x 64 lanes x 4 (accumulator order), then z.
  static constexpr int SLOT_USED = NTILE * 256 + DF;
  static constexpr int SLOT = (SLOT_USED + 63) / 64 * 64;
  static constexpr bool fits = lds_fwd <= kMaxLds;
};

// Per-head decay: g = a, b = 1 - a (eqs 10-11); g = b = 1 without decay.
struct Decay {
  float g, b, lg;
  __device__ Decay(const float *decay, int h) {
    g = decay ? decay[h] : 1.f;
    b = decay ? 1.f - g : 1.f;
    lg = log2f(g);
  }
};

// Registers holding one [C][W] slab of a [n][W] row-major matrix, as 16-byte
// pieces distributed over the 256 threads (consecutive threads, consecutive
// pieces: fully coalesced).
template <typename T, int W, int C>
struct Slab {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int PPR = W / VEC;                 // pieces per row
  static constexpr int PIECES = C * PPR;
  static constexpr int PER = (PIECES + kThreads - 1) / kThreads;
  uint4 v[PER];

  __device__ __forceinline__ void load(const T *base, int64_t row0, int rows,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + kThreads * i;
      const int row = p / PPR, col = (p % PPR) * VEC;
      v[i] = make_uint4(0, 0, 0, 0);
      if (p < PIECES && row < rows)
        v[i] = *reinterpret_cast<const uint4 *>(base + (row0 + row) * W + col);
    }
  }
};

// phi(x) on the fp32 value of a stored element.
__device__ __forceinline__ float feat(float x, int elu1) {
  return elu1 ? elu_plus_one(x) : x;
}

// Write phi(Q) rows into sQ (row-major, rows >= r zeroed).
template <typename T, int W, int C, int L>
__device__ __forceinline__ void stage_rowmajor(const Slab<T, W, C> &sl, T *dst,
                                               int rows, int tid, int elu1) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      Vec16<T> x, y;
      x.raw = sl.v[i];
#pragma unroll
      for (int e = 0; e < S::VEC; ++e) {
        const float f = row < rows ? feat(to_f32(x.e[e]), elu1) : 0.f;
        y.e[e] = from_f32<T>(f);
      }
      *reinterpret_cast<uint4 *>(dst + row * L + col) = y.raw;
    }
  }
}

// Write phi(K) rows into sK (row-major, unweighted) and, weighted by
// w_s = b g^(r-1-s), transposed into sKT.  Rows >= r are zero in both.
template <typename T, int W, int C, int LQ, int LT, bool ROWMAJOR>
__device__ __forceinline__ void stage_keys(const Slab<T, W, C> &sl, T *sK,
                                           T *sKT, const float *gp, float b,
                                           int rows, int tid, int elu1) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      const float w = row < rows ? b * gp[rows - 1 - row] : 0.f;
      Vec16<T> x, y;
      x.raw = sl.v[i];
#pragma unroll
      for (int e = 0; e < S::VEC; ++e) {
        const float f = row < rows ? feat(to_f32(x.e[e]), elu1) : 0.f;
        y.e[e] = from_f32<T>(f);
        sKT[(col + e) * LT + row] = from_f32<T>(f * w);
      }
      if (ROWMAJOR) *reinterpret_cast<uint4 *>(sK + row * LQ + col) = y.raw;
    }
  }
}

// Write V rows transposed into sVT (rows >= r zero).
template <typename T, int W, int C, int LT>
__device__ __forceinline__ void stage_values(const Slab<T, W, C> &sl, T *sVT,
                                             int rows, int tid) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      Vec16<T> x;
      x.raw = sl.v[i];
#pragma unroll
      for (int e = 0; e < S::VEC; ++e)
        sVT[(col + e) * LT + row] = row < rows ? x.e[e] : from_f32<T>(0.f);
    }
  }
}

// S tile (fb, jb) += (w.K')^T V over the chunk:  A = sKT rows f, B = sVT rows j,
// contraction over the chunk positions s (contiguous k-assignment).
template <typename T, int C, int LT>
__device__ __forceinline__ f32x4 state_tile_update(f32x4 acc, const T *sKT,
                                                   const T *sVT, int fb, int jb,
                                                   int li, int g) {
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    Frag<T> a, bb;
    load_frag8(a, sKT + (16 * fb + li) * LT + 32 * kb + 8 * g);
    load_frag8(bb, sVT + (16 * jb + li) * LT + 32 * kb + 8 * g);
    acc = mma(a, bb, acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Kernel 1: segment aggregates (end state of each segment from zero).
// ---------------------------------------------------------------------------
template <typename T, int D, int DF>
__global__ __launch_bounds__(kThreads) void la_agg_kernel(FwdArgs a) {
  using F = FwdShape<T, D, DF>;
  constexpr int C = F::C, LT = F::LT;
  extern __shared__ __align__(16) unsigned char smem[];
  T *sKT = reinterpret_cast<T *>(smem);
  T *sVT = sKT + F::SKT;
  float *gp = reinterpret_cast<float *>(sVT + F::SVT);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t unit = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const Decay dk(a.decay, static_cast<int>(unit % a.H));
  for (int i = tid; i <= C; i += kThreads) gp[i] = pow_int(dk.g, dk.lg, i);

  const T *kb = static_cast<const T *>(a.k) + unit * a.n * DF;
  const T *vb = static_cast<const T *>(a.v) + unit * a.n * D;
  const int64_t start = seg * a.seg_len;
  const int64_t end = min(a.n, start + a.seg_len);

  f32x4 S[F::TPW];
#pragma unroll
  for (int i = 0; i < F::TPW; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float z = 0.f;

  Slab<T, DF, C> rk;
  Slab<T, D, C> rv;
  rk.load(kb, start, static_cast<int>(min<int64_t>(C, end - start)), tid);
  rv.load(vb, start, static_cast<int>(min<int64_t>(C, end - start)), tid);
  __syncthreads();  // gp ready
  for (int64_t row0 = start; row0 < end; row0 += C) {
    const int rows = static_cast<int>(min<int64_t>(C, end - row0));
    stage_keys<T, DF, C, F::LQ, LT, false>(rk, nullptr, sKT, gp, dk.b, rows,
                                           tid, a.elu1);
    stage_values<T, D, C, LT>(rv, sVT, rows, tid);
    __syncthreads();
    if (row0 + C < end) {
      const int r2 = static_cast<int>(min<int64_t>(C, end - row0 - C));
      rk.load(kb, row0 + C, r2, tid);
      rv.load(vb, row0 + C, r2, tid);
    }
    const float gr = gp[rows];
#pragma unroll
    for (int i = 0; i < F::TPW; ++i) {
      const int idx = w + kWaves * i;
      if (idx < F::NTILE)
        S[i] = state_tile_update<T, C, LT>(S[i] * gr, sKT, sVT, idx / F::NJ,
                                           idx % F::NJ, li, g);
    }
    if (tid < DF) {
      float zs = 0.f;
      for (int s = 0; s < C; ++s) zs += to_f32(sKT[tid * LT + s]);
      z = gr * z + zs;
    }
    __syncthreads();
  }
  float *slot = a.states + (unit * (a.nseg + 1) + seg) * F::SLOT;
#pragma unroll
  for (int i = 0; i < F::TPW; ++i) {
    const int idx = w + kWaves * i;
    if (idx < F::NTILE)
      *reinterpret_cast<f32x4 *>(slot + (idx * 64 + lane) * 4) = S[i];
  }
  if (tid < DF) slot[F::NTILE * 256 + tid] = z;
}

// ---------------------------------------------------------------------------
// Kernel 3: chunked forward of one segment from its entering state.
// ---------------------------------------------------------------------------
template <typename T, int D, int DF, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void la_fwd_kernel(FwdArgs a) {
  using F = FwdShape<T, D, DF>;
  constexpr int C = F::C, LQ = F::LQ, LT = F::LT, LS = F::LS, DFP = F::DFP;
  constexpr int STRIPS = F::STRIPS, NJ = F::NJ;
  extern __shared__ __align__(16) unsigned char smem[];
  T *sQ = reinterpret_cast<T *>(smem);
  T *sK = sQ + F::SQ;
  T *sKT = sK + F::SK;
  T *sVT = sKT + F::SKT;
  T *sST = sVT + F::SVT;
  float *sz = reinterpret_cast<float *>(sST + F::SST);
  float *gp = sz + DF;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t unit = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const Decay dk(a.decay, static_cast<int>(unit % a.H));
  for (int i = tid; i <= C; i += kThreads) gp[i] = pow_int(dk.g, dk.lg, i);

  const T *qb = static_cast<const T *>(a.q) + unit * a.n * DF;
  const T *kb = static_cast<const T *>(a.k) + unit * a.n * DF;
  const T *vb = static_cast<const T *>(a.v) + unit * a.n * D;
  T *ob = static_cast<T *>(a.out) + unit * a.n * D;
  const int64_t start = seg * a.seg_len;
  const int64_t end = min(a.n, start + a.seg_len);

  // Zero the k-padding columns of q', k' and S^T once (DF < 32 only).
  if (DFP != DF) {
    for (int i = tid; i < C * (DFP - DF); i += kThreads) {
      const int row = i / (DFP - DF), col = DF + i % (DFP - DF);
      sQ[row * LQ + col] = from_f32<T>(0.f);
      sK[row * LQ + col] = from_f32<T>(0.f);
    }
    for (int i = tid; i < D * (DFP - DF); i += kThreads)
      sST[(i / (DFP - DF)) * LS + DF + i % (DFP - DF)] = from_f32<T>(0.f);
  }

  // Entering state: exclusive prefix (causal) or total (non-causal).
  const float *st = nullptr;
  if (a.states)
    st = a.states + (unit * (a.nseg + 1) + (CAUSAL ? seg : a.nseg)) * F::SLOT;
  f32x4 S[F::TPW];
#pragma unroll
  for (int i = 0; i < F::TPW; ++i) {
    const int idx = w + kWaves * i;
    S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (idx < F::NTILE) {
      if (st) S[i] = *reinterpret_cast<const f32x4 *>(st + (idx * 64 + lane) * 4);
      const int fb = idx / NJ, jb = idx % NJ;
      store4(sST + (16 * jb + li) * LS + 16 * fb + 4 * g, S[i][0], S[i][1],
             S[i][2], S[i][3]);
    }
  }
  for (int f = tid; f < DF; f += kThreads) sz[f] = st ? st[F::NTILE * 256 + f] : 0.f;

  Slab<T, DF, C> rq, rk;
  Slab<T, D, C> rv;
  {
    const int r0 = static_cast<int>(min<int64_t>(C, end - start));
    rq.load(qb, start, r0, tid);
    if (CAUSAL) {
      rk.load(kb, start, r0, tid);
      rv.load(vb, start, r0, tid);
    }
  }
  __syncthreads();  // gp, sST, sz ready

  for (int64_t row0 = start; row0 < end; row0 += C) {
    const int rows = static_cast<int>(min<int64_t>(C, end - row0));
    const bool last = row0 + C >= end;
    stage_rowmajor<T, DF, C, LQ>(rq, sQ, rows, tid, a.elu1);
    if (CAUSAL) {
      stage_keys<T, DF, C, LQ, LT, true>(rk, sK, sKT, gp, dk.b, rows, tid,
                                         a.elu1);
      stage_values<T, D, C, LT>(rv, sVT, rows, tid);
    }
    __syncthreads();  // operand tiles ready
    if (!last) {
      const int r2 = static_cast<int>(min<int64_t>(C, end - row0 - C));
      rq.load(qb, row0 + C, r2, tid);
      if (CAUSAL) {
        rk.load(kb, row0 + C, r2, tid);
        rv.load(vb, row0 + C, r2, tid);
      }
    }

    // ---- readout of this wave's strips ----
    for (int tb = w; tb < STRIPS; tb += kWaves) {
      const int t = 16 * tb + li;
      f32x4 pt[STRIPS];
      float den_i = 0.f;
#pragma unroll
      for (int sb = 0; sb < STRIPS; ++sb) {
        pt[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (CAUSAL && sb <= tb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kq = 0; kq < DFP / 32; ++kq) {
            Frag<T> fa, fb;
            load_frag8(fa, sK + (16 * sb + li) * LQ + 32 * kq + 8 * g);
            load_frag8(fb, sQ + (16 * tb + li) * LQ + 32 * kq + 8 * g);
            acc = mma(fa, fb, acc);
          }
          // acc[rr] = q'_t . k'_s with s = 16 sb + 4 g + rr
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int s = 16 * sb + 4 * g + rr;
            const float wgt = s <= t ? dk.b * gp[t - s] : 0.f;
            acc[rr] = round_to<T>(acc[rr] * wgt);
            den_i += acc[rr];
          }
          pt[sb] = acc;
        }
      }
      constexpr int NPK = (STRIPS + 1) / 2;
      Frag<T> pf[NPK];
#pragma unroll
      for (int kp = 0; kp < NPK; ++kp)
        frag_from_acc(pf[kp], pt[2 * kp],
                      2 * kp + 1 < STRIPS ? pt[2 * kp + 1]
                                          : f32x4{0.f, 0.f, 0.f, 0.f});
      den_i = wave_sum_groups(den_i);
      float dx = 0.f;
#pragma unroll
      for (int ff = 0; ff < DF / 4; ++ff) {
        const int f = g * (DF / 4) + ff;
        dx += to_f32(sQ[t * LQ + f]) * sz[f];
      }
      dx = wave_sum_groups(dx);
      const float gt = CAUSAL ? gp[t + 1] : 1.f;
      const float den = den_i + gt * dx;
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
        if (CAUSAL) {
#pragma unroll
          for (int kp = 0; kp < NPK; ++kp) {
            if (2 * kp <= tb) {
              Frag<T> fa;
              const T *row = sVT + (16 * jb + li) * LT + 32 * kp;
              load_frag44(fa, row + 4 * g, row + 16 + 4 * g);
              an = mma(fa, pf[kp], an);
            }
          }
        }
#pragma unroll
        for (int kq = 0; kq < DFP / 32; ++kq) {
          Frag<T> fa, fb;
          load_frag8(fa, sST + (16 * jb + li) * LS + 32 * kq + 8 * g);
          load_frag8(fb, sQ + (16 * tb + li) * LQ + 32 * kq + 8 * g);
          ai = mma(fa, fb, ai);
        }
        // an[rr], ai[rr]: column j = 16 jb + 4 g + rr of output row t
        if (t < rows)
          store4(ob + (row0 + t) * D + 16 * jb + 4 * g,
                 (an[0] + gt * ai[0]) / den, (an[1] + gt * ai[1]) / den,
                 (an[2] + gt * ai[2]) / den, (an[3] + gt * ai[3]) / den);
      }
    }

    if (CAUSAL && !last) {
      // ---- state update: S <- g^r S + (w.K')^T V, z <- g^r z + sum w k' ----
      const float gr = gp[rows];
#pragma unroll
      for (int i = 0; i < F::TPW; ++i) {
        const int idx = w + kWaves * i;
        if (idx < F::NTILE)
          S[i] = state_tile_update<T, C, LT>(S[i] * gr, sKT, sVT, idx / NJ,
                                             idx % NJ, li, g);
      }
      float znew = 0.f;
      if (tid < DF) {
        float zs = 0.f;
        for (int s = 0; s < C; ++s) zs += to_f32(sKT[tid * LT + s]);
        znew = gr * sz[tid] + zs;
      }
      __syncthreads();  // every wave has finished reading sST, sz, sQ, sK
#pragma unroll
      for (int i = 0; i < F::TPW; ++i) {
        const int idx = w + kWaves * i;
        if (idx < F::NTILE) {
          const int fb = idx / NJ, jb = idx % NJ;
          store4(sST + (16 * jb + li) * LS + 16 * fb + 4 * g, S[i][0], S[i][1],
                 S[i][2], S[i][3]);
        }
      }
      if (tid < DF) sz[tid] = znew;
    } else {
      __syncthreads();  // before the next chunk overwrites the tiles
    }
  }
}

}  // namespace la
