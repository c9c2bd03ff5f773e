// Chunked forward with a decay per state row (gfx950).
//
// The gated recurrence with one decay per feature row f of the state,
//   mu_t[f][:] = g_t[f] mu_{t-1}[f][:] + (1 - g_t[f]) k'_t[f] v_t,
//   nu_t[f]    = g_t[f] nu_{t-1}[f]    + (1 - g_t[f]) k'_t[f],
//   out_t      = q'_t mu_t / q'_t . nu_t,
// with g_t[f] = exp(lam[f]) (the diagonal A of "2.3 State-Space Models" eqs
// 21-25 on the efficient2 page: one decay per row and head, the same at every
// position) or g_t[f] = exp(lam_t[f]) (an input-dependent decay per position
// and row, the selective dA = exp(A delta_t) of the "Linear attention
// research 2026" page, Mamba section, applied row-wise).  Causal readout is
// the causal form of "2.2 Linear Attention" eq 9; the non-causal readout uses
// the sums after the last position.
//
// Chunks of kRowC = 16 positions, one matrix-core tile high.  With L_t[f]
// the log2 of the decay accumulated from the chunk's start through row t:
//   inter-chunk readout:  num_t += (q'_t * 2^L_t) mu_prev
//   state carry:          mu_next = 2^L_15 mu_prev
//                                   + sum_s (k'_s (1-g_s) 2^(L_15-L_s))^T v_s
//   intra-chunk scores:   P[t][s] = sum_f q'_t[f] k'_s[f] (1-g_s[f])
//                                   2^(L_t[f] - L_s[f]),  s <= t,
// the first two with factors at most 1; the last has its weight inside the
// sum over f.  For s < t it is split about an anchor row a with s <= a < t:
//   P[t][s] = (q'_t * 2^(L_t - L_a)) . (k'_s (1-g_s) 2^(L_a - L_s)),
// both factors at most 1, so neither overflows, and one underflows only
// where the weight itself is below 2^-126.  The anchor comes from the
// highest bit b in which s and t differ (a binary hierarchy over the 16
// rows): level b holds, in one tile, every row r as a key (bit b of r
// clear) or as a query (bit b set) about a = r with bits 0..b-1 set and bit
// b clear, so s (a key) and t (a query) of the same block meet at the same
// a.  Four products (b = 3, 2, 1, 0), each tile both operands, and each
// score taken from its level; the diagonal P[t][t] = sum_f q'_t k'_t
// (1 - g_t) has no decay factor and is summed in fp32 by the scaling role.
// Inside the scores only, a step's log2 decay is floored at kRowFloor (a
// step that forgets more than all but 2^-32 of its past is taken to forget
// exactly that), which keeps the sums finite for log decays of -inf.
//
// Work split of a workgroup (4 waves, one segment of one (batch, head) unit):
//   * scaling role, every thread: row t = lane % 16 of the chunk and groups
//     of 8 features j = lane / 16 + 4 wave (+ 16 per iteration); it loads
//     q, k (and the decay) of its row and features, applies phi, forms the
//     scaled operands into LDS, the partial denominator q~ . nu and
//     diagonal score, and keeps nu (replicated over the 16 row lanes) up to
//     date;
//   * matrix role, wave w: value column blocks jb = w, w + 4, ...; it keeps
//     those columns of the fp32 state in its accumulators (rows f = 16 i +
//     4 (lane / 16) + r, column 16 jb + lane % 16), which feed the readout
//     directly as operands ("split" k-assignment), and forms P^T itself.
// One barrier per chunk: the scaling of chunk c + 1 fills the other LDS
// buffer while the matrix role works on chunk c (where two buffers do not
// fit, one buffer and a second barrier).
//
// Segments of a unit run as separate workgroups in three launches: the
// aggregates (each segment's state from zero, its nu and its summed log2
// decay per row), a scan that turns them into each segment's incoming state
// (and the total), then the readout from that state.  No workgroup waits for
// another.
#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kRowC = kRowChunk;
constexpr int kRowThreads = 256;
constexpr float kRowFloor = -32.f;
constexpr float kLog2E = 1.4426950408889634f;

template <typename T, int D, int DF>
struct RowShape {
  static constexpr int DFP = DF < 32 ? 32 : DF;  // contraction width (zero pad)
  static constexpr int NFT = DFP / 16;           // state row tiles
  static constexpr int NKB = DFP / 32;           // 32-wide k blocks over f
  static constexpr int NEB = D / 16;             // value column blocks
  static constexpr int EPW = (NEB + 3) / 4;      // column blocks per wave
  static constexpr int NG = DFP / 8;             // 8-feature groups per row
  static constexpr int NIT = (NG + 15) / 16;     // groups per scaling thread
  // Row strides by how a tile is read.  Q~ and the score tiles give each lane a row
  // (8-byte reads at column 4 (lane / 16)): a stride of 8 (mod 32) bf16
  // elements spreads 16 rows x 2 column groups over all 64 banks.  K~ and V
  // are read transposed (ds_read_b64_tr_b16: 4 rows x 4 column quads per
  // 16 lanes), which wants 16 (mod 32).  fp32 tiles: 4 floats of padding.
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int PADT = sizeof(T) == 2 ? 16 : 4;
  static constexpr int LQ = DFP + PAD;           // Q~, Q^, K^ row stride
  static constexpr int LT = DFP + PADT;          // K~ row stride
  static constexpr int LV = D % 32 == 16 && sizeof(T) == 2 ? D : D + PADT;
  static constexpr int TILE = kRowC * LQ;        // elements per operand tile
  static constexpr int VE = 16 / static_cast<int>(sizeof(T));  // per 16 B
  static constexpr int NVG = kRowC * D / VE;     // 16-byte value groups
  // tiles: Q~, four score levels (row stride LQ), K~ (LT), V (LV), then the
  // per-wave partial denominators and diagonal scores, the chunk's decay
  static constexpr int OFF_V = (5 * TILE + kRowC * LT) * static_cast<int>(sizeof(T));
  static constexpr int OFF_DEN = OFF_V + kRowC * LV * static_cast<int>(sizeof(T));
  static constexpr int OFF_DIAG = OFF_DEN + 4 * kRowC * 4;
  static constexpr int OFF_DEC = OFF_DIAG + 4 * kRowC * 4;
  static constexpr int BUF = OFF_DEC + DFP * 4;
  // two LDS buffers (scaling of the next chunk overlaps the products of
  // this one) where they fit, else one (fp32, d' = 256) and a second
  // barrier per chunk
  static constexpr int NB = 2 * BUF <= 160 * 1024 ? 2 : 1;
  static constexpr int lds_bytes = NB * BUF;
  // aggregate slot: state in accumulator order, then nu, then sum log2 g
  static constexpr int NSTATE = NEB * NFT * 256;
  static constexpr int SLOT = NSTATE + 2 * DFP;
  static_assert(BUF % 16 == 0, "LDS buffers stay 16-byte aligned");
};

// ---------------------------------------------------------------------------
// K = 16 matrix-core fragments: lane l holds k = 4 (l / 16) + e, e = 0..3.
// ---------------------------------------------------------------------------
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { s16x4 v; };
template <> struct Frag16<float> { float v[4]; };

__device__ __forceinline__ f32x4 mma16(const Frag16<bf16> &a,
                                       const Frag16<bf16> &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag16<float> &a,
                                       const Frag16<float> &b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// Rows r0 .. r0 + 3 of column n0 + i of a row-major tile (stride ld).
__device__ __forceinline__ void tr16(Frag16<bf16> &f, const bf16 *base, int ld,
                                     int r0, int n0, int i) {
  f.v = ds_read_tr4(base + (r0 + i / 4) * ld + n0 + 4 * (i % 4));
}
__device__ __forceinline__ void tr16(Frag16<float> &f, const float *base,
                                     int ld, int r0, int n0, int i) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[e] = base[(r0 + e) * ld + n0 + i];
}

// A K = 16 fragment as a K = 32 one ("split" assignment: k = 4 (l / 16) + e
// from f, k = 16 + 4 (l / 16) + e zero).  A 16x16x16 bf16 product must not
// accumulate onto the result of a 16x16x32 one issued less than 8 wait
// states before it (it then reads a stale accumulator; measured), and the
// compiler places them back to back, so products that chain onto a K = 32
// accumulation are widened to K = 32 with a zero half instead.
__device__ __forceinline__ void frag_widen(Frag<bf16> &w, const Frag16<bf16> &f) {
  const u32x2 u = __builtin_bit_cast(u32x2, f.v);
  const u32x4 x = {u[0], u[1], 0u, 0u};
  w.v = __builtin_bit_cast(bf16x8, x);
}
__device__ __forceinline__ void frag_widen(Frag<float> &w, const Frag16<float> &f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w.v[e] = f.v[e];
    w.v[4 + e] = 0.f;
  }
}

// Accumulator column slice (rows 4 (l / 16) + e) as a K = 16 fragment.
__device__ __forceinline__ void frag16_from_acc(Frag16<bf16> &f,
                                                const f32x4 &a) {
  const u32x2 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  f.v = __builtin_bit_cast(s16x4, u);
}
__device__ __forceinline__ void frag16_from_acc(Frag16<float> &f,
                                                const f32x4 &a) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[e] = a[e];
}
__device__ __forceinline__ float frag16_sum(const Frag16<bf16> &f) {
  const u32x2 u = __builtin_bit_cast(u32x2, f.v);
  return (bf16_lo(u[0]) + bf16_hi(u[0])) + (bf16_lo(u[1]) + bf16_hi(u[1]));
}
__device__ __forceinline__ float frag16_sum(const Frag16<float> &f) {
  return (f.v[0] + f.v[1]) + (f.v[2] + f.v[3]);
}

// ---------------------------------------------------------------------------
// 16-lane row operations (DPP within each row of 16 lanes).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float row_dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xf, 0xf, true));
}
// Inclusive prefix sum over lanes 0..t of the row (row_shr fills zeros).
__device__ __forceinline__ float row_prefix(float x) {
  x += row_dpp<0x111>(x);
  x += row_dpp<0x112>(x);
  x += row_dpp<0x114>(x);
  x += row_dpp<0x118>(x);
  return x;
}
// Sum over lanes t + 1 .. 15 of the row (row_shl fills zeros).
__device__ __forceinline__ float row_suffix_excl(float x) {
  x = row_dpp<0x101>(x);
  x += row_dpp<0x101>(x);
  x += row_dpp<0x102>(x);
  x += row_dpp<0x104>(x);
  x += row_dpp<0x108>(x);
  return x;
}
// Sum over the whole row, in every lane (rotations).
__device__ __forceinline__ float row_sum(float x) {
  x += row_dpp<0x128>(x);
  x += row_dpp<0x124>(x);
  x += row_dpp<0x122>(x);
  x += row_dpp<0x121>(x);
  return x;
}

// ---------------------------------------------------------------------------
// Per-element factors of one scaling thread (row t, 8 features).
// ---------------------------------------------------------------------------
struct RowFac {
  float qt[8];   // readout operand:  2^L_t
  float x[4][8]; // score operand of level b = 3 - i: as a key (bit b of t
                 // clear) (1 - g_t) 2^(Lf_a - Lf_t), as a query 2^(Lf_t - Lf_a)
  float b[8];    // 1 - g_t (diagonal score)
  float kt[8];   // carry operand:    (1 - g_t) 2^(L_15 - L_t)
  float tot[8];  // L_15 (log2 decay of the whole chunk)
  float dec[8];  // 2^L_15
};

// c * l with 0 * (-inf) taken as 0 (no step, no decay).
__device__ __forceinline__ float steps_log2(int c, float l) {
  return c == 0 ? 0.f : static_cast<float>(c) * l;
}

// One decay per row (the same at every position): closed forms in the
// number of live rows before and at t (rows past `rows` are padding: no
// decay, no input).
__device__ __forceinline__ void channel_factors(RowFac &F, const float (&l)[8],
                                                const float (&b)[8], int t,
                                                int rows) {
  const int cnt = t + 1 < rows ? t + 1 : rows;
  const bool live = t < rows;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float lf = fmaxf(l[e], kRowFloor);
    F.qt[e] = __builtin_amdgcn_exp2f(steps_log2(cnt, l[e]));
    F.b[e] = live ? b[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bit = 3 - i, lo = (1 << bit) - 1;
      const int an = (t & ~(2 * lo + 1)) | lo;       // anchor row
      const int ca = an + 1 < rows ? an + 1 : rows;  // live rows through it
      const bool key = ((t >> bit) & 1) == 0;
      // |live rows between the anchor and t| steps of decay, at most 1
      const float ex = static_cast<float>(key ? ca - cnt : cnt - ca) * lf;
      F.x[i][e] = key ? (live ? b[e] * __builtin_amdgcn_exp2f(ex) : 0.f)
                      : __builtin_amdgcn_exp2f(ex);
    }
    F.kt[e] = live ? b[e] * __builtin_amdgcn_exp2f(steps_log2(rows - cnt, l[e]))
                   : 0.f;
    F.tot[e] = steps_log2(rows, l[e]);
    F.dec[e] = __builtin_amdgcn_exp2f(F.tot[e]);
  }
}

// One decay per position and row: scans over the 16 rows of the chunk (the
// lanes of this thread's 16-lane row).  Padding rows carry l = 0, b = 0.
__device__ __forceinline__ void position_factors(RowFac &F, const float (&l)[8],
                                                 const float (&b)[8], int t,
                                                 int lane) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = row_prefix(l[e]);
    const float lf = fmaxf(l[e], kRowFloor);
    const float pf = row_prefix(lf);
    const float sx = row_suffix_excl(l[e]);
    F.tot[e] = row_sum(l[e]);
    F.qt[e] = __builtin_amdgcn_exp2f(p);
    F.b[e] = b[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bit = 3 - i, lo = (1 << bit) - 1;
      const int an = (t & ~(2 * lo + 1)) | lo;
      const float pa = __shfl(pf, (lane & ~15) | an);  // prefix at the anchor
      const bool key = ((t >> bit) & 1) == 0;
      F.x[i][e] = key ? b[e] * __builtin_amdgcn_exp2f(pa - pf)
                      : __builtin_amdgcn_exp2f(pf - pa);
    }
    F.kt[e] = b[e] * __builtin_amdgcn_exp2f(sx);
    F.dec[e] = __builtin_amdgcn_exp2f(F.tot[e]);
  }
}

// ---------------------------------------------------------------------------
// 8 consecutive elements of type T: raw 16-byte words and conversions.
// ---------------------------------------------------------------------------
template <typename T> struct Raw8 {
  static constexpr int W = static_cast<int>(sizeof(T)) / 2;  // 16-byte words
  u32x4 r[W];
};
template <typename T>
__device__ __forceinline__ void raw8_load(Raw8<T> &x, __amdgpu_buffer_rsrc_t rs,
                                          unsigned off) {
#pragma unroll
  for (int w = 0; w < Raw8<T>::W; ++w) x.r[w] = buffer_load16(rs, off + 16u * w);
}
__device__ __forceinline__ void raw8_float(const Raw8<bf16> &x, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(x.r[0][e]);
    f[2 * e + 1] = bf16_hi(x.r[0][e]);
  }
}
// (whole-vector reinterpretation: per-element bit casts of an ext-vector are
// not reliable with this compiler)
__device__ __forceinline__ void raw8_float(const Raw8<float> &x, float (&f)[8]) {
  const f32x4 a = __builtin_bit_cast(f32x4, x.r[0]);
  const f32x4 b = __builtin_bit_cast(f32x4, x.r[1]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = a[e];
    f[4 + e] = b[e];
  }
}
// Round 8 values to T, store them at p (16-byte aligned) and hand back the
// rounded values.
__device__ __forceinline__ void store8(bf16 *p, float (&x)[8]) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    x[2 * e] = bf16_lo(u[e]);
    x[2 * e + 1] = bf16_hi(u[e]);
  }
  *reinterpret_cast<u32x4 *>(p) = u;
}
__device__ __forceinline__ void store8(float *p, float (&x)[8]) {
  const f32x4 a = {x[0], x[1], x[2], x[3]}, c = {x[4], x[5], x[6], x[7]};
  reinterpret_cast<f32x4 *>(p)[0] = a;
  reinterpret_cast<f32x4 *>(p)[1] = c;
}

// PHASE 0: causal readout; 1: segment aggregates; 2: non-causal readout.
// PP: the decay is given per position and row (else per row only; the
// non-causal readout reads no decay).
// Two waves per SIMD where the state fits beside them (bf16 operands,
// d' <= 128): the chunk loop is a chain of dependent steps, and a second
// workgroup per CU hides their latency.
template <typename T, int D, int DF, int PHASE, bool PP>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(
    sizeof(T) == 2 && DF <= 128 ? 2 : 1))) void la_fwd_rows_kernel(RowArgs a) {
  using S = RowShape<T, D, DF>;
  constexpr int DFP = S::DFP, NFT = S::NFT, NKB = S::NKB, NEB = S::NEB,
                EPW = S::EPW, NG = S::NG, NIT = S::NIT, LQ = S::LQ, LT = S::LT,
                LV = S::LV;
  constexpr bool READ = PHASE != 1;   // forms outputs
  constexpr bool CARRY = PHASE != 2;  // runs the recurrence through the chunk
  constexpr bool SCORE = PHASE == 0;  // intra-chunk scores
  constexpr unsigned ES = sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int64_t unit = blockIdx.x / a.nseg;
  const int seg = static_cast<int>(blockIdx.x % a.nseg);
  if (PHASE == 1 && a.skip_last && seg == a.nseg - 1) return;
  const int h = static_cast<int>(unit % a.H);
  const int64_t start = seg * a.seg_len;
  const int64_t end = start + a.seg_len < a.n ? start + a.seg_len : a.n;
  const int nch = static_cast<int>((end - start + kRowC - 1) / kRowC);
  const T *qg = static_cast<const T *>(a.q) + unit * a.n * DF;
  const T *kg = static_cast<const T *>(a.k) + unit * a.n * DF;
  const T *vg = static_cast<const T *>(a.v) + unit * a.n * D;
  T *og = static_cast<T *>(a.out) + unit * a.n * D;
  const float *lg = PP ? a.lam + unit * a.n * DF : a.lam + h * DF;
  float *slot0 = a.agg ? a.agg + unit * (a.nseg + 1) * static_cast<int64_t>(S::SLOT)
                       : nullptr;

  // ---- scaling role state -------------------------------------------------
  const int t = i16;
  // log2 g and 1 - g of this thread's features (one decay per row; padding
  // features: no decay, no input)
  auto channel_decay = [&](int j, float (&l)[8], float (&b)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float lam = 8 * j < DF ? a.lam[h * DF + 8 * j + e] : 0.f;
      l[e] = lam * kLog2E;
      b[e] = -expm1f(lam);
    }
  };
  float nu[NIT][8];       // nu of this thread's features (same in all 16 rows)
  float dsum[NIT][8];     // summed log2 decay of the segment (per position)
  float rr[NIT][8];       // aggregates: decay from the chunk's end to the
                          // segment's end (chunks run last to first)
  RowFac fc[NIT];         // one decay per row: factors of a full chunk
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int j = g + 4 * w + 16 * it;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      nu[it][e] = 0.f;
      dsum[it][e] = 0.f;
      rr[it][e] = 1.f;
    }
    if (CARRY && !PP && j < NG) {
      float l[8], b[8];
      channel_decay(j, l, b);
      channel_factors(fc[it], l, b, t, kRowC);
    }
  }

  // ---- matrix role state --------------------------------------------------
  f32x4 st[EPW][NFT];
#pragma unroll
  for (int m = 0; m < EPW; ++m)
#pragma unroll
    for (int i = 0; i < NFT; ++i) st[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Incoming state: this segment's carry (causal) or the total (non-causal).
  if (PHASE == 2 || (PHASE == 0 && a.nseg > 1)) {
    const float *sl = slot0 + (PHASE == 2 ? a.nseg : seg) * static_cast<int64_t>(S::SLOT);
#pragma unroll
    for (int m = 0; m < EPW; ++m) {
      const int jb = w + 4 * m;
      if (jb < NEB) {
#pragma unroll
        for (int i = 0; i < NFT; ++i)
          st[m][i] = reinterpret_cast<const f32x4 *>(sl)[(jb * NFT + i) * 64 + lane];
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = g + 4 * w + 16 * it;
      if (j < NG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) nu[it][e] = sl[S::NSTATE + 8 * j + e];
      }
    }
  }

  // ---- chunk loads (registers) -------------------------------------------
  Raw8<T> rq[NIT], rk[NIT];
  Raw8<float> rl[NIT];
  constexpr int NVI = (S::NVG + kRowThreads - 1) / kRowThreads;
  u32x4 rv[NVI];
  auto rows_of = [&](int c) {
    const int64_t r = end - (start + static_cast<int64_t>(c) * kRowC);
    return r < kRowC ? static_cast<int>(r) : kRowC;
  };
  auto issue = [&](int c) {
    const int64_t r0 = start + static_cast<int64_t>(c) * kRowC;
    const unsigned rows = static_cast<unsigned>(rows_of(c));
    const __amdgpu_buffer_rsrc_t rsq = make_rsrc(qg + r0 * DF, rows * DF * ES);
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(kg + r0 * DF, rows * DF * ES);
    const __amdgpu_buffer_rsrc_t rsl =
        make_rsrc(lg + r0 * DF, PP ? rows * DF * 4u : 0u);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = g + 4 * w + 16 * it;
      const unsigned off = (t * DF + 8 * j) * ES;
      const bool in = j < NG && 8 * j < DF;
      if (READ) {
        if (in) raw8_load(rq[it], rsq, off);
        else for (int x = 0; x < Raw8<T>::W; ++x) rq[it].r[x] = u32x4{0, 0, 0, 0};
      }
      if (CARRY) {
        if (in) raw8_load(rk[it], rsk, off);
        else for (int x = 0; x < Raw8<T>::W; ++x) rk[it].r[x] = u32x4{0, 0, 0, 0};
        if (PP && in)
          raw8_load(rl[it], rsl, (t * DF + 8 * j) * 4u);
        else
          for (int x = 0; x < 2; ++x) rl[it].r[x] = u32x4{0, 0, 0, 0};
      }
    }
    if (CARRY) {
      const __amdgpu_buffer_rsrc_t rsv = make_rsrc(vg + r0 * D, rows * D * ES);
#pragma unroll
      for (int x = 0; x < NVI; ++x) {
        const int idx = tid + kRowThreads * x;
        const int row = idx / (D / S::VE), cg = idx % (D / S::VE);
        rv[x] = idx < S::NVG ? buffer_load16(rsv, (row * D + cg * S::VE) * ES)
                             : u32x4{0, 0, 0, 0};
      }
    }
  };

  // ---- scaling role: chunk c into LDS buffer b ----------------------------
  auto scale = [&](int c, int b) {
    unsigned char *buf = smem + b * S::BUF;
    T *QT = reinterpret_cast<T *>(buf);
    T *XS = QT + S::TILE, *KT = QT + 5 * S::TILE;  // four score tiles
    T *VV = reinterpret_cast<T *>(buf + S::OFF_V);
    float *DENP = reinterpret_cast<float *>(buf + S::OFF_DEN);
    float *DIAGP = reinterpret_cast<float *>(buf + S::OFF_DIAG);
    float *DEC = reinterpret_cast<float *>(buf + S::OFF_DEC);
    const int rows = rows_of(c);
    float den = 0.f, dg = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = g + 4 * w + 16 * it;
      if (j >= NG) continue;
      const int f0 = 8 * j;
      const bool in = f0 < DF;
      RowFac F;
      float qv[8];  // phi(q) of this row's features (also for the diagonal)
      if (CARRY) {
        if constexpr (PP) {
          float l[8], bb[8];
          raw8_float(rl[it], l);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bb[e] = -expm1f(l[e]);
            l[e] *= kLog2E;
          }
          position_factors(F, l, bb, t, lane);
        } else if (rows < kRowC) {
          float l[8], bb[8];
          channel_decay(j, l, bb);
          channel_factors(F, l, bb, t, rows);
        } else {
          F = fc[it];
        }
      }
      if (READ) {
        float x[8];
        raw8_float(rq[it], qv);
        if (a.elu1 && in)
          for (int e = 0; e < 8; ++e) qv[e] = elu_plus_one_fast(qv[e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = CARRY ? qv[e] * F.qt[e] : qv[e];
        store8(QT + t * LQ + f0, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) den += x[e] * nu[it][e];
        if (SCORE) {
          // as a query at the levels where bit (3 - i) of t is set
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((t >> (3 - i)) & 1) {
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = qv[e] * F.x[i][e];
              store8(XS + i * S::TILE + t * LQ + f0, x);
            }
        }
      }
      if (CARRY) {
        float kv[8], x[8];
        raw8_float(rk[it], kv);
        if (a.elu1 && in)
          for (int e = 0; e < 8; ++e) kv[e] = elu_plus_one_fast(kv[e]);
        if (SCORE) {
          // as a key at the others; and the diagonal score's part
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (((t >> (3 - i)) & 1) == 0) {
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = kv[e] * F.x[i][e];
              store8(XS + i * S::TILE + t * LQ + f0, x);
            }
#pragma unroll
          for (int e = 0; e < 8; ++e) dg += qv[e] * kv[e] * F.b[e];
        }
        if constexpr (PHASE == 1) {
          // aggregates run the chunks last to first: each chunk's carry
          // operand takes the decay still to come in the segment, so the
          // state and nu are plain sums (no per-chunk decay of the state);
          // each lane sums its own row's part of nu, and the rows are
          // summed once, after the last chunk
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = kv[e] * (F.kt[e] * rr[it][e]);
          store8(KT + t * LT + f0, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            nu[it][e] += x[e];
            rr[it][e] *= F.dec[e];
            if (PP) dsum[it][e] += F.tot[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = kv[e] * F.kt[e];
          store8(KT + t * LT + f0, x);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            nu[it][e] = F.dec[e] * nu[it][e] + row_sum(x[e]);
        }
        if (PHASE == 0 && t == 0) {
          const f32x4 d0 = {F.dec[0], F.dec[1], F.dec[2], F.dec[3]};
          const f32x4 d1 = {F.dec[4], F.dec[5], F.dec[6], F.dec[7]};
          reinterpret_cast<f32x4 *>(DEC + f0)[0] = d0;
          reinterpret_cast<f32x4 *>(DEC + f0)[1] = d1;
        }
      }
    }
    if (READ) {
      den = wave_sum_groups(den);
      if (g == 0) DENP[w * kRowC + t] = den;
      if (SCORE) {
        dg = wave_sum_groups(dg);
        if (g == 0) DIAGP[w * kRowC + t] = dg;
      }
    }
    if (CARRY) {
#pragma unroll
      for (int x = 0; x < NVI; ++x) {
        const int idx = tid + kRowThreads * x;
        if (idx < S::NVG) {
          const int row = idx / (D / S::VE), cg = idx % (D / S::VE);
          *reinterpret_cast<u32x4 *>(VV + row * LV + cg * S::VE) = rv[x];
        }
      }
    }
  };

  // ---- matrix role: chunk c from LDS buffer b -----------------------------
  auto matrix = [&](int c, int b) {
    if (w >= NEB) return;
    const unsigned char *buf = smem + b * S::BUF;
    const T *QT = reinterpret_cast<const T *>(buf);
    const T *XS = QT + S::TILE, *KT = QT + 5 * S::TILE;
    const T *VV = reinterpret_cast<const T *>(buf + S::OFF_V);
    const float *DENP = reinterpret_cast<const float *>(buf + S::OFF_DEN);
    const float *DIAGP = reinterpret_cast<const float *>(buf + S::OFF_DIAG);
    const float *DEC = reinterpret_cast<const float *>(buf + S::OFF_DEC);
    const int rows = rows_of(c);
    const int64_t r0 = start + static_cast<int64_t>(c) * kRowC;

    Frag16<T> pf;
    float dr[4];
    if (READ) {
      float den = (DENP[t] + DENP[kRowC + t]) + (DENP[2 * kRowC + t] + DENP[3 * kRowC + t]);
      if (SCORE) {
        // P^T: rows s = 4 g + r, column t = lane % 16; keep s <= t.  Level
        // i's tile is both operands of its product (keys and queries in
        // different rows); entry (t, s < t) comes from the level of the
        // highest bit in which s and t differ, the diagonal from the
        // scaling role's fp32 sums.
        f32x4 pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pl[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            Frag<T> fx;
            const T *xs = XS + i * S::TILE + i16 * LQ + 32 * kb;
            load_frag44(fx, xs + 4 * g, xs + 16 + 4 * g);
            pl[i] = mma(fx, fx, pl[i]);
          }
        }
        const float dg = (DIAGP[t] + DIAGP[kRowC + t]) +
                         (DIAGP[2 * kRowC + t] + DIAGP[3 * kRowC + t]);
        f32x4 pt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sr = 4 * g + r, x = sr ^ i16;
          pt[r] = sr > i16 ? 0.f
                  : x == 0 ? dg
                  : x >= 8 ? pl[0][r]
                  : x >= 4 ? pl[1][r]
                  : x >= 2 ? pl[2][r] : pl[3][r];
        }
        frag16_from_acc(pf, pt);
        den += wave_sum_groups(frag16_sum(pf));
      }
      // reciprocal of each output row's denominator (hardware, within
      // 1 ulp: far below the storage rounding that follows)
      const float rden = __builtin_amdgcn_rcpf(den);
#pragma unroll
      for (int r = 0; r < 4; ++r) dr[r] = __shfl(rden, 4 * g + r);
    }

#pragma unroll
    for (int m = 0; m < EPW; ++m) {
      const int jb = w + 4 * m;
      if (jb >= NEB) break;
      Frag16<T> vf;
      if (CARRY) tr16(vf, VV, LV, 4 * g, 16 * jb, i16);
      if (READ) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          Frag<T> fa, fs;
          load_frag44(fa, QT + i16 * LQ + 32 * kb + 4 * g,
                      QT + i16 * LQ + 32 * kb + 16 + 4 * g);
          frag_from_acc(fs, st[m][2 * kb], st[m][2 * kb + 1]);
          acc = mma(fa, fs, acc);
        }
        if (SCORE) {  // + P V, widened to K = 32 (see frag_widen)
          Frag<T> pw, vw;
          frag_widen(pw, pf);
          frag_widen(vw, vf);
          acc = mma(pw, vw, acc);
        }
        T *o = og + (r0 + 4 * g) * D + 16 * jb + i16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < rows) o[r * D] = from_f32<T>(acc[r] * dr[r]);
      }
      if (CARRY) {
#pragma unroll
        for (int i = 0; i < NFT; ++i) {
          Frag16<T> kf;
          tr16(kf, KT, LT, 4 * g, 16 * i, i16);
          if constexpr (PHASE == 1) {
            st[m][i] = mma16(kf, vf, st[m][i]);
          } else {
            const f32x4 dc = *reinterpret_cast<const f32x4 *>(DEC + 16 * i + 4 * g);
            f32x4 s0 = st[m][i];
#pragma unroll
            for (int r = 0; r < 4; ++r) s0[r] *= dc[r];
            st[m][i] = mma16(kf, vf, s0);
          }
        }
      }
    }
  };

  // ---- chunk loop: one barrier per chunk ----------------------------------
  // (step i handles chunk i; the aggregates take chunk nch - 1 - i)
  auto chunk_at = [&](int i) { return PHASE == 1 ? nch - 1 - i : i; };
  constexpr int NB = S::NB;
  issue(chunk_at(0));
  scale(chunk_at(0), 0);
  for (int i = 0; i < nch; ++i) {
    __syncthreads();
    if (i + 1 < nch) issue(chunk_at(i + 1));
    matrix(chunk_at(i), NB == 2 ? i & 1 : 0);
    if (i + 1 < nch) {
      if (NB == 1) __syncthreads();  // one buffer: its readers are done
      scale(chunk_at(i + 1), NB == 2 ? (i + 1) & 1 : 0);
    }
  }

  // ---- results ------------------------------------------------------------
  if (PHASE == 1) {
    float *sl = slot0 + seg * static_cast<int64_t>(S::SLOT);
#pragma unroll
    for (int m = 0; m < EPW; ++m) {
      const int jb = w + 4 * m;
      if (jb < NEB) {
#pragma unroll
        for (int i = 0; i < NFT; ++i)
          reinterpret_cast<f32x4 *>(sl)[(jb * NFT + i) * 64 + lane] = st[m][i];
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int e = 0; e < 8; ++e) nu[it][e] = row_sum(nu[it][e]);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = g + 4 * w + 16 * it;
      if (j < NG && t == 0) {
        if (!PP) {  // one decay per row: the segment's rows times log2 g
          float l[8], b[8];
          channel_decay(j, l, b);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            dsum[it][e] = steps_log2(static_cast<int>(end - start), l[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sl[S::NSTATE + 8 * j + e] = nu[it][e];
          sl[S::NSTATE + DFP + 8 * j + e] = dsum[it][e];
        }
      }
    }
  }
  if (PHASE == 0 && a.mu_out && seg == a.nseg - 1) {
#pragma unroll
    for (int m = 0; m < EPW; ++m) {
      const int jb = w + 4 * m;
      if (jb < NEB) {
#pragma unroll
        for (int i = 0; i < NFT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int f = 16 * i + 4 * g + r;
            if (f < DF) a.mu_out[(unit * DF + f) * D + 16 * jb + i16] = st[m][i][r];
          }
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = g + 4 * w + 16 * it;
      if (j < NG && t == 0 && 8 * j < DF)
        for (int e = 0; e < 8; ++e) a.nu_out[unit * DF + 8 * j + e] = nu[it][e];
    }
  }
}

}  // namespace la
