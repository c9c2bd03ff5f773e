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
// Unrolling eqs 10-11 from a state S gives mu_t = g^(t+1) S + sum_{s<=t}
// b g^(t-s) k'_s^T v_s, which the first three lines read out, and the state
// after the chunk, the last two.  Without decay every weight is 1 (eqs 7-8).
// The normaliser z is eq 8 = eq 7 with v = 1: V is extended by a block of 16
// columns holding (1, 0, ..., 0), so the state tiles of that block carry z in
// their first column and the matrix cores update and read it with S.
//
// One fused kernel, one 512-thread workgroup (8 waves) per sequence segment:
//   phase 1 (several segments per (batch, head) unit only): the segment's
//     aggregate, i.e. its end state from a zero state, from K and V alone,
//     written to the workspace;
//   exchange: each segment publishes its aggregate and a flag in its unit's
//     line of the workspace, waits for the flags of the segments it needs
//     (those before it; all of them when non-causal) and sums their
//     aggregates, weighted by the decay over the gap, into the state entering
//     it.  Only workgroups of one unit wait on each other.  Causal segments
//     are numbered in the order their workgroups start, so every wait is on
//     a running workgroup.  Non-causal segments need every aggregate: they
//     run as two launches instead (aggregates, then readout), so nothing
//     waits inside a kernel;
//   phase 2: the chunk loop from that state.
// Both loops keep several chunks of loads in flight in a register ring.  All
// global loads are unconditional (tail rows clamp to a valid row; the loop
// runs whole ring revolutions, padding with empty chunks) so the compiler's
// wait before each chunk only covers that chunk's loads.
//
// LDS tiles are all row-major ([position][feature]), written with 16-byte
// stores; operands whose contraction index runs along rows are read with the
// transposing LDS read (see la_device.h).  Row strides are 16 mod 32 bf16
// elements, which makes those reads bank-conflict free.
//
// Work split per chunk (phase 2):
//   - staging: every thread takes 16-byte pieces of Q, K, V; phi in fp32 for
//     Q and K; K' rows past the end are zeroed (they feed the state; Q and V
//     tails only reach outputs that are never stored);
//   - readout: output strip tb (16 rows) belongs to waves tb and tb + STRIPS,
//     which split its 16-column blocks; each forms the strip's P^T on the
//     matrix cores and feeds the accumulator straight back as the B operand
//     of V^T P^T ("split" k-assignment); S^T Q'^T comes from a T copy of S^T
//     in LDS, and its extra block gives q'_t . z;
//   - state: fp32 16x16 accumulator tiles spread over the waves, each chunk
//     adding (w.K')^T [V | 1] on the matrix cores.
#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kMaxLds = 160 * 1024;

// Registers holding one [C][W] slab of a [n][W] row-major matrix as 16-byte
// pieces; consecutive threads take consecutive pieces (coalesced).
template <typename T, int W, int C>
struct Slab {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int PPR = W / VEC;                 // pieces per row
  static constexpr int PIECES = C * PPR;
  static constexpr int PER = (PIECES + kThreads - 1) / kThreads;
  static constexpr bool EXACT = PIECES % kThreads == 0;
  u32x4 v[PER];

  // Rows row0 .. row0 + rows - 1 of base; pieces of later rows read zero
  // (the resource ends after the last valid row, so those rows cost no
  // memory traffic).  Piece p of the slab sits at byte 16 p.
  __device__ __forceinline__ void load(const T *base, int64_t row0, int rows,
                                       int tid) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(
        base + row0 * W, static_cast<unsigned>(rows) * W * sizeof(T));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + kThreads * i;
      if (EXACT || p < PIECES) v[i] = buffer_load16(r, 16u * p);
    }
  }
  // The same W columns out of rows of ld >= W elements (a column part of a
  // wider matrix); the resource ends after the last valid row's W columns.
  __device__ __forceinline__ void load_ld(const T *base, int64_t row0,
                                          int rows, int ld, int tid) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(
        base + row0 * ld,
        rows > 0 ? static_cast<unsigned>((rows - 1) * ld + W) * sizeof(T) : 0u);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + kThreads * i;
      if (EXACT || p < PIECES)
        v[i] = buffer_load16(
            r, static_cast<unsigned>((p / PPR) * ld + (p % PPR) * VEC) *
                   sizeof(T));
    }
  }
};

// Row stride (elements) for a row of w elements: 16 mod 32 for bf16 (the
// transposing reads of 8 rows then hit disjoint banks), +4 for fp32.
template <typename T>
constexpr int lds_stride(int w) {
  return sizeof(T) == 2 ? (w % 32 == 16 ? w : w + 16) : w + 4;
}

// Feature map an instance applies to q and k while staging them.
constexpr int kMapFeatures = 0;   // q, k are features already
constexpr int kMapElu = 1;        // elu + 1 (d' = d)
constexpr int kMapPerformer = 2;  // Performer random features, fused

// LDS bytes of one instance with chunk length c (see FwdShape): nbuf sets of
// the q', w.k' (wkeys) and V tiles, nst S^T copies (0: one per set), kslots
// slots of k', the raw q, k rows of the fused Performer map, and per set a
// table of tab floats (the chunk's decay weights, where the instance keeps
// one).
template <typename T>
constexpr size_t fwd_lds_bytes(int c, int d, int df, bool wkeys, bool pf,
                               int kslots = 1, int nbuf = 1, int tab = 0,
                               int nst = 0) {
  const int dfp = df < 32 ? 32 : df;
  const size_t sq = static_cast<size_t>(c) * lds_stride<T>(dfp);
  const size_t sv = static_cast<size_t>(c) * lds_stride<T>(d + 16);
  const size_t sst = static_cast<size_t>(d + 16) * lds_stride<T>(dfp);
  const size_t sx = pf ? static_cast<size_t>(c) * lds_stride<T>(d) : 0;
  return sizeof(T) * (nbuf * (sq + (wkeys ? sq : 0) + sv) +
                      (nst > 0 ? nst : nbuf) * sst + kslots * sq + 2 * sx) +
         sizeof(float) * (c + 8 + kMaxSegments + (pf ? 2 * c : 0) + nbuf * tab);
}

// Largest power of two <= x, at most 8 (1 for x < 2).
constexpr int pow2_floor(int x) {
  return x >= 8 ? 8 : x >= 4 ? 4 : x >= 2 ? 2 : 1;
}

// DK: 0 no decay (eqs 7-8); 1 one decay a per head (eqs 10-11); 2 a decay
// per position, given as its natural log (the input-dependent decay).
template <typename T, int D, int DF, int DK, int MAP = kMapFeatures>
struct FwdShape {
  static constexpr bool DECAY = DK != 0;
  static constexpr bool SEL = DK == 2;    // per-position decay
  static constexpr bool PF = MAP == kMapPerformer;
  static constexpr int DV = D;                       // value width d
  // width of the q, k rows in memory: d for the fused Performer map
  static constexpr int QW = PF ? D : DF;
  // Chunk rows: 64 for bf16 operands; 32 where LDS would not hold 64.
  static constexpr int C =
      PF ? (fwd_lds_bytes<T>(64, D, DF, DK == 1, true, 1, 1,
                             SEL ? 3 * 64 + 4 : 0) <= kMaxLds
                ? 64
                : 32)
         : ((sizeof(T) == 2 && !(DF == 256 && D == 128)) ? 64 : 32);
  // Floats of one tile set's table: per-position decay, see sel_table; one
  // decay per head with register weights (RW, below), the state-update
  // weight of each key.  WOFF: where those weights start.
  static constexpr int TABW = SEL ? 3 * C + 4 : 0;
  static constexpr int TABR = SEL ? 3 * C + 4 : DK == 1 ? C : 0;
  static constexpr int WOFF = SEL ? 2 * C : 0;
  static constexpr int DFP = DF < 32 ? 32 : DF;      // padded k-width of q', k'
  static constexpr int LQ = lds_stride<T>(DFP);      // sQ, sK, sKw, sST
  static constexpr int LV = lds_stride<T>(D + 16);   // sV: V | ones block
  static constexpr int LX = lds_stride<T>(D);        // raw q, k rows
  static constexpr int STRIPS = C / 16;
  static constexpr int WPS = kWaves / STRIPS;        // waves per output strip
  static constexpr int NJ = D / 16, NF = DF / 16;
  static constexpr int NJA = NJ + 1;                 // with the ones block
  static constexpr int NTILE = NF * NJA;             // 16x16 state tiles
  // state tiles of a wave: see tile_fb / tile_jb
  static constexpr int FPW = NF >= kWaves ? NF / kWaves : 1;
  static constexpr int WPF = NF >= kWaves ? 1 : kWaves / NF;
  static constexpr int JPW = (NJA + WPF - 1) / WPF;
  static constexpr int SQ = C * LQ, SV = C * LV, SST = (D + 16) * LQ,
                       SX = PF ? C * LX : 0;
  // Fused Performer projection: omega^T tiles per wave (kept in registers
  // for the whole kernel) and the strips each wave maps.  NF >= 8: wave w
  // owns feature tiles w + 8 m for every strip; else tile w % NF for strips
  // w / NF + WPT j (WPT waves per tile).
  static constexpr int TPW = NF >= kWaves ? NF / kWaves : 1;
  static constexpr int WPT = NF >= kWaves ? 1 : kWaves / NF;
  static constexpr int SPW = (STRIPS + WPT - 1) / WPT;
  // Software pipelining (both loops): two sets of operand tiles, so that
  // chunk c + 1 is mapped and staged while chunk c is multiplied; where LDS
  // holds the second set.  With two S^T copies as well the chunk loop has
  // one barrier; with one (NST = 1, where only that fits) the state is
  // published between two barriers, and the staging still overlaps the
  // matrix work.
  // Resident keys (bf16, no decay, d, d' <= 64): phase 1 keeps phi(K) of each
  // chunk of a short segment (at most KRES_ chunks) in its own slot of sK and
  // phase 2 reuses it instead of loading and mapping K again.
  static constexpr bool RES_OK =
      !PF && !DECAY && sizeof(T) == 2 && D <= 64 && DF <= 64;
  static constexpr int KRES_ =
      !RES_OK ? 0
      : fwd_lds_bytes<T>(C, D, DF, false, PF, 8, 2) <= kMaxLds ? 8
      : fwd_lds_bytes<T>(C, D, DF, false, PF, 4, 2) <= kMaxLds ? 4
                                                           : 0;
  static constexpr int KS2 = KRES_ > 2 ? KRES_ : 2;
  // candidate layouts: pipelined with a weighted key tile (one decay per
  // head), pipelined without one, with one or two S^T copies
  static constexpr bool PIPE_W =
      !PF && DK == 1 &&
      fwd_lds_bytes<T>(C, D, DF, true, PF, KS2, 2, TABW) <= kMaxLds;
  static constexpr bool PIPE_R2 =
      !PF && fwd_lds_bytes<T>(C, D, DF, false, PF, KS2, 2, TABR) <= kMaxLds;
  // (not with per-position decay: its chunk loop measured 1 % slower so at
  // d = d' = 128)
  static constexpr bool PIPE_R1 =
      !PF && !SEL &&
      fwd_lds_bytes<T>(C, D, DF, false, PF, KS2, 2, TABR, 1) <= kMaxLds;
  // One decay per head: the state update reads a staged tile of weighted
  // keys (WKEYS) where that layout is pipelined, or where nothing is and
  // LDS holds the tile; else (RW) it weights the key fragments in registers
  // from a per-chunk table, as per-position decay does.
  static constexpr bool WKEYS =
      DK == 1 && (PF || PIPE_W ||
                  (!PIPE_R2 && !PIPE_R1 &&
                   fwd_lds_bytes<T>(C, D, DF, true, false, 1, 1, TABW) <=
                       kMaxLds));
  static constexpr bool RW = DK == 1 && !WKEYS;
  static constexpr int SKW = WKEYS ? C * LQ : 0;
  static constexpr int TAB = WKEYS ? TABW : TABR;
  static constexpr bool PIPE = WKEYS ? PIPE_W : (PIPE_R2 || PIPE_R1);
  static constexpr int NBUF = PIPE ? 2 : 1;                 // sets of tiles
  static constexpr int NST = PIPE && (WKEYS || PIPE_R2) ? 2 : 1;  // S^T copies
  static constexpr int KS = PIPE ? KS2 : 1;                 // slots of sK
  static constexpr size_t lds_bytes =
      fwd_lds_bytes<T>(C, D, DF, WKEYS, PF, KS, NBUF, TAB, NST);
  // fp32 state slot: NTILE tiles x 64 lanes x 4 (accumulator order).
  static constexpr int SLOT = NTILE * 256;
  // Workgroups per compute unit the instance is built for: two (<= 128
  // VGPRs, 4 waves per SIMD) for the small bf16 shapes where LDS holds two,
  // else one.
  static constexpr int OCC = (!PF && sizeof(T) == 2 && D <= 64 && DF <= 64 &&
                              2 * lds_bytes <= kMaxLds)
                                 ? 2
                                 : 1;
  static_assert(OCC * kCUs <= kMaxTargetGroups, "sync area too small");
  static constexpr int WAVES_PER_SIMD = OCC * kWaves / 4;
  // Register-ring depths: chunks of loads in flight per workgroup.  With
  // every CU streaming, shallow rings measured fastest: more loads in flight
  // only made each chunk's data arrive later.  Phase 1 (K, V) keeps the
  // next chunk in flight; phase 2 (q, k, v) the next two where a chunk's
  // loads take at most 24 VGPRs (bf16 d <= 128: 1 % faster at d = 128 than
  // one chunk), else the next one.
  static constexpr int REG2 = 4 * (Slab<T, QW, C>::PER * 2 + Slab<T, D, C>::PER);
  static constexpr int NB2 = REG2 <= 24 ? 2 : 1;
  static constexpr int NB1 = 1;
  static constexpr int KRES = PIPE ? KRES_ : 0;
  // the fused Performer map needs bf16 operands, d a multiple of 32 (the
  // projection's k-width), at least 32 features, and d d' <= 128 * 128 (the
  // register budget of one workgroup per CU; larger shapes spill)
  static constexpr bool fits =
      lds_bytes <= kMaxLds &&
      (!PF || (sizeof(T) == 2 && D % 32 == 0 && DF >= 32 && D * DF <= 16384));
};

// State tile ownership: wave w holds tiles (fb, jb) with
//   fb = w % NF (NF < 8) or w + 8 m (NF >= 8),
//   jb = w / NF + WPF m' (NF < 8) or every jb (NF >= 8).
// Where that jb would be past the last block, the wave holds a copy of tile
// (fb, NJA - 1) instead: every wave then runs the same instructions, and the
// copy, computed from the same operands in the same order, is bitwise equal
// to the original, so writing it out again is harmless.
template <typename F>
__device__ __forceinline__ int tile_fb(int w, int m) {
  return F::NF >= kWaves ? w + kWaves * m : w % F::NF;
}
template <typename F>
__device__ __forceinline__ int tile_jb(int w, int m) {
  return F::NF >= kWaves ? m : min(w / F::NF + F::WPF * m, F::NJA - 1);
}
// Whether state tile m of wave w is a copy of another wave's ones-block
// tile (dup), or the ones-block tile whose copies other waves hold (owner).
template <typename F>
__device__ __forceinline__ bool dup_tile(int w, int m) {
  return F::NF < kWaves && w / F::NF + F::WPF * m > F::NJA - 1;
}
template <typename F>
__device__ __forceinline__ bool owns_ones_tile(int w, int m) {
  return F::NF < kWaves && w / F::NF + F::WPF * m == F::NJA - 1;
}
// Whether a wave's state tile m is the ones block (or its copy) in every
// wave, which the tile layout fixes at compile time.
template <typename F>
__device__ __forceinline__ constexpr bool ones_tile(int m) {
  return F::NF >= kWaves ? m == F::NJ : F::WPF * m >= F::NJ;
}
// A V (or V^T) fragment of the ones block in any lane assignment: lane
// (g, i) holds column D + i, which is 1 for i = 0, 4, 8, 12 at every row.
template <typename T>
__device__ __forceinline__ Frag<T> ones_frag(int li) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = from_f32<T>(li % 4 == 0 ? 1.f : 0.f);
  return f;
}

// ---------------------------------------------------------------------------
// Per-position decay (the input-dependent decay of the Mamba section of the
// "Linear attention research 2026" page, applied as eqs 10-11 with a per
// position: gamma_t = exp(lam_t), input weight 1 - gamma_t).  With L_t the
// sum of log2 gamma over the chunk's rows 0..t, the chunk formulas weight
//   P[t][s] by (1 - gamma_s) 2^(L_t - L_s)   (s <= t),
//   the entering state's readout by 2^(L_t),
//   key s in the state update by (1 - gamma_s) 2^(L_last - L_s),
//   the state itself by 2^(L_last),
// where L_last is the sum over the whole chunk (rows past the end have
// lam = 0).
// ---------------------------------------------------------------------------

// The chunk's log decays, one per row, in the first C threads (one dword
// each, so a partly valid 16-byte piece can never be dropped whole by the
// range check); 0 past the valid rows and in the other threads.
template <int C>
struct LamSlab {
  float v;
  __device__ __forceinline__ void load(const float *base, int64_t row0,
                                       int rows, int tid) {
    v = 0.f;
    if (tid < C) {
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(base + row0, static_cast<unsigned>(rows) * 4u);
      v = __builtin_bit_cast(float,
                             __builtin_amdgcn_raw_buffer_load_b32(r, 4u * tid, 0, 0));
    }
  }
};

// The chunk's table, computed by the threads of wave 0 from their LamSlab
// (C <= 64, lane t holds row t): tab[t] = L_t, tab[C + t] = 1 - gamma_t,
// tab[2C + t] = state-update weight of key t, tab[3C] = 2^(L_last).  Returns
// L_last (every lane).
template <int C>
__device__ __forceinline__ float sel_table(float lam, float *tab, int lane) {
  static_assert(C <= kWave, "one row per lane of one wave");
  constexpr float kLog2e = 1.4426950408889634f;
  // Below -104, exp(lam) is 0 in fp32 (under the smallest subnormal), so
  // the floor changes no decay; it keeps the sums finite when lam = -inf
  // (a full reset), whose differences would otherwise be -inf - -inf.
  lam = fmaxf(lam, -104.f);
  float L = lane < C ? lam * kLog2e : 0.f;
#pragma unroll
  for (int o = 1; o < C; o <<= 1) {  // inclusive scan over the chunk's rows
    const float y = __shfl_up(L, o);
    if (lane >= o) L += y;
  }
  const float last = __shfl(L, C - 1);
  if (lane < C) {
    const float beta = -expm1f(lam);  // 1 - gamma, accurate for gamma near 1
    tab[lane] = L;
    tab[C + lane] = beta;
    tab[2 * C + lane] = beta * __builtin_amdgcn_exp2f(last - L);
    if (lane == 0) tab[3 * C] = __builtin_amdgcn_exp2f(last);
  }
  return last;
}

// One decay per head with the weights in registers (RW): the state-update
// weight b g^(rows-1-s) of each key s of the chunk, 0 past the valid rows,
// written by the first C lanes of one wave.
template <int C>
__device__ __forceinline__ void rw_table(float *tab, const float *gp, float b,
                                         int rows, int lane) {
  if (lane < C) tab[lane] = lane < rows ? b * gp[rows - 1 - lane] : 0.f;
}

// Per-head decay: g = a, b = 1 - a (eqs 10-11); g = b = 1 without decay.
struct Decay {
  float g, b, lg;
  __device__ Decay(const float *decay, int h) {
    g = decay ? decay[h] : 1.f;
    b = decay ? 1.f - g : 1.f;
    lg = log2f(g);
  }
};

// phi over one 16-byte piece of T values (elu + 1 in fp32 when ELU, else the
// values themselves), times w when SCALE, rounded once to T.
template <typename T, bool ELU, bool SCALE>
__device__ __forceinline__ u32x4 phi_piece(const u32x4 &x, float w) {
  if constexpr (!ELU && !SCALE) {
    return x;
  } else {
    auto f = [&](float v) {
      const float y = ELU ? elu_plus_one_fast(v) : v;
      return SCALE ? y * w : y;
    };
    if constexpr (sizeof(T) == 2) {
      u32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] = pack_bf16x2(f(bf16_lo(x[i])), f(bf16_hi(x[i])));
      return y;
    } else {
      // whole-vector reinterpretation (per-element bit casts of vector
      // elements are not reliable with this compiler)
      const f32x4 xf = __builtin_bit_cast(f32x4, x);
      const f32x4 yf = {f(xf[0]), f(xf[1]), f(xf[2]), f(xf[3])};
      return __builtin_bit_cast(u32x4, yf);
    }
  }
}

// phi(Q) rows -> sQ (row-major).  Rows past the end are staged unmasked: they
// only reach outputs that are never stored.
template <typename T, int W, int C, int L, bool ELU>
__device__ __forceinline__ void stage_queries(const Slab<T, W, C> &sl, T *dst,
                                              int tid) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (S::EXACT || p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      *reinterpret_cast<u32x4 *>(dst + row * L + col) =
          phi_piece<T, ELU, false>(sl.v[i], 1.f);
    }
  }
}

// phi(K) rows -> sK (row-major, when PLAIN), zero past the end (a bit mask on
// the packed result, no branch); the keys the state update uses go to sKw:
// w_s phi(k_s) with w_s = b g^(rows-1-s) under decay (sKw is then its own
// tile), else sKw aliases sK.  Tail rows hold a copy of a valid row, so every
// masked value is finite.
template <typename T, int W, int C, int L, bool DECAY, bool PLAIN, bool ELU>
__device__ __forceinline__ void stage_keys(const Slab<T, W, C> &sl, T *sK,
                                           T *sKw, const float *gp, float b,
                                           int rows, int tid) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (S::EXACT || p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      const bool valid = row < rows;
      const unsigned m = valid ? ~0u : 0u;
      const u32x4 mm = {m, m, m, m};
      if (DECAY) {
        const float w = b * gp[valid ? rows - 1 - row : 0];
        if (PLAIN)
          *reinterpret_cast<u32x4 *>(sK + row * L + col) =
              phi_piece<T, ELU, false>(sl.v[i], 1.f) & mm;
        *reinterpret_cast<u32x4 *>(sKw + row * L + col) =
            phi_piece<T, ELU, true>(sl.v[i], w) & mm;
      } else {
        *reinterpret_cast<u32x4 *>(sK + row * L + col) =
            phi_piece<T, ELU, false>(sl.v[i], 1.f) & mm;
      }
    }
  }
}

// V rows -> sV (row-major, raw copy: tail rows meet zero keys or dropped rows).
template <typename T, int W, int C, int L>
__device__ __forceinline__ void stage_values(const Slab<T, W, C> &sl, T *sV,
                                             int tid) {
  using S = Slab<T, W, C>;
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    if (S::EXACT || p < S::PIECES) {
      const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
      *reinterpret_cast<u32x4 *>(sV + row * L + col) = sl.v[i];
    }
  }
}

// x moved from lane l ^ 1, l ^ 2 (quad permutations), or mirrored within
// 8 or 16 lanes (DPP row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf,
                                      0xf, false));
}
// Sum over aligned groups of N = 4, 8 or 16 consecutive lanes.
template <int N>
__device__ __forceinline__ float sum_lane_groups(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "lane group");
  x += dpp_f32<0xb1>(x);                    // quad_perm 1, 0, 3, 2
  x += dpp_f32<0x4e>(x);                    // quad_perm 2, 3, 0, 1
  if constexpr (N >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}

// Raw q or k rows of one chunk for the fused Performer map -> sX
// (row-major), and for each row the exponent offset of its features,
// c0 = -|x|^2 log2(e) / 2 - log2 sqrt(m), to c0[row]: -inf for rows at or
// past valid_rows, whose features are then exactly 0.  The PPR threads that
// stage a row's pieces sum their squares in fp32 and combine them across
// lanes, so every norm is computed once per chunk.
template <typename T, int W, int C, int L>
__device__ __forceinline__ void stage_rows_pf(const Slab<T, W, C> &sl, T *sX,
                                              float *c0, float lsm,
                                              int valid_rows, int tid) {
  using S = Slab<T, W, C>;
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(sizeof(T) == 2, "bf16 rows");
#pragma unroll
  for (int i = 0; i < S::PER; ++i) {
    const int p = tid + kThreads * i;
    const bool mine = S::EXACT || p < S::PIECES;
    const int row = p / S::PPR, col = (p % S::PPR) * S::VEC;
    float n = 0.f;
    if (mine) {
      *reinterpret_cast<u32x4 *>(sX + row * L + col) = sl.v[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16_lo(sl.v[i][k]), hi = bf16_hi(sl.v[i][k]);
        n += lo * lo + hi * hi;
      }
    }
    n = sum_lane_groups<S::PPR>(n);
    if (mine && p % S::PPR == 0)
      c0[row] = row < valid_rows ? -0.5f * kLog2e * n - lsm : -__builtin_inff();
  }
}

// Performer features of the rows of one chunk, fused ("Linear attention
// research 2026" page, Performer random features: phi(x) = exp(x omega -
// |x|^2 / 2) / sqrt(m)).  u^T = omega^T X^T runs on the matrix cores: A =
// this wave's omega^T tiles (registers, see FwdShape::TPW), B = the raw q or
// k rows (LDS), contraction over d.  The omega tiles carry the factor
// log2 e and each accumulator starts at its row's exponent offset c0 (see
// stage_rows_pf; c0q for the queries, c0k for the keys), so for each feature
// tile fb the accumulator of row 16 ts + li holds the base-2 exponents of
// features 16 fb + 4 g .. +3: one exp2 per feature, stored as 4 consecutive
// values.  WQ maps the queries into dq; WK maps the keys: rows >= rows are
// zero (c0 = -inf), and under decay the weighted copy w_s phi(k_s),
// w_s = b g^(rows-1-s), goes to dkw (the plain one to dk when PLAIN or
// without decay).
template <typename F, typename T, bool WQ, bool WK, bool DECAY, bool PLAIN>
__device__ __forceinline__ void performer_features(
    const Frag<T> (&wf)[F::TPW][F::DV / 32], const T *sXq, const T *sXk,
    const float *c0q, const float *c0k, T *dq, T *dk, T *dkw,
    const float *gp, float b, int rows, int w, int g, int li) {
  constexpr int KB = F::DV / 32;  // k-blocks of the contraction over d
#pragma unroll
  for (int j = 0; j < F::SPW; ++j) {
    const int ts = F::NF >= kWaves ? j : w / F::NF + F::WPT * j;
    if (ts < F::STRIPS) {
      const int row = 16 * ts + li;
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        const bool keys = mat == 1;
        if ((keys && WK) || (!keys && WQ)) {
          Frag<T> xf[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            load_frag8(xf[kb],
                       (keys ? sXk : sXq) + row * F::LX + 32 * kb + 8 * g);
          const float c0 = (keys ? c0k : c0q)[row];
          const float wr = (keys && DECAY)
                               ? (row < rows ? b * gp[rows - 1 - row] : 0.f)
                               : 1.f;
#pragma unroll
          for (int m = 0; m < F::TPW; ++m) {
            const int fb = F::NF >= kWaves ? w + kWaves * m : w % F::NF;
            f32x4 acc = {c0, c0, c0, c0};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc = mma(wf[m][kb], xf[kb], acc);
            float ph[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ph[r] = __builtin_amdgcn_exp2f(acc[r]);
            const int off = row * F::LQ + 16 * fb + 4 * g;
            if (!keys) {
              store4(dq + off, ph[0], ph[1], ph[2], ph[3]);
            } else {
              if (!DECAY || PLAIN) store4(dk + off, ph[0], ph[1], ph[2], ph[3]);
              if (DECAY)
                store4(dkw + off, ph[0] * wr, ph[1] * wr, ph[2] * wr,
                       ph[3] * wr);
            }
          }
        }
      }
    }
  }
}

// S tiles of this wave += (w.K')^T [V | 1] over the chunk: A = rows of sKw
// read transposed (features along lanes), B = rows of sV read transposed
// (columns along lanes); contraction over the chunk positions.
// kmask = 0 drops the keys (the state is only scaled by gr).  With wk (per-
// position decay) the keys of sKw are plain and position s is weighted by
// wk[s] in registers.
template <typename F, typename T>
__device__ __forceinline__ void state_update(f32x4 *S, const T *sKw,
                                             const T *sV, float gr, int w,
                                             int g, int li,
                                             unsigned kmask = ~0u,
                                             const float *wk = nullptr) {
  constexpr int C = F::C;
#pragma unroll
  for (int m = 0; m < F::FPW; ++m) {
    const int fb = tile_fb<F>(w, m);
    Frag<T> af[C / 32];
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      load_frag_tr8(af[kb], sKw, F::LQ, 32 * kb, 16 * fb, g, li);
      frag_mask(af[kb], u32x4{kmask, kmask, kmask, kmask});
      if constexpr (F::SEL || F::RW) {  // positions 32 kb + 8 g + e
        const f32x4 *wp = reinterpret_cast<const f32x4 *>(wk + 32 * kb + 8 * g);
        frag_scale(af[kb], wp[0], wp[1]);
      }
    }
#pragma unroll
    for (int mj = 0; mj < F::JPW; ++mj) {
      const int jb = tile_jb<F>(w, mj);
      f32x4 acc = S[m * F::JPW + mj] * gr;
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        Frag<T> bf;
        if (ones_tile<F>(mj))  // a constant, not read from LDS
          bf = ones_frag<T>(li);
        else
          load_frag_tr8(bf, sV, F::LV, 32 * kb, 16 * jb, g, li);
        acc = mma(af[kb], bf, acc);
      }
      S[m * F::JPW + mj] = acc;
    }
  }
}

// Column of S^T element (row, col) in sST.  With bf16 tiles, rows whose bit
// 2 is set swap their 16-byte pieces in pairs: that spreads the 8-byte state
// writes below over more banks (measured on gfx950 with 8 waves: 64 instead
// of 112 cycles per write at a 160-byte row stride) while the 16-byte
// fragment reads of the readout stay conflict-free.  Groups of 4 and 8
// aligned columns stay together.
template <typename T>
__device__ __forceinline__ int sst_col(int row, int col) {
  return sizeof(T) == 2 ? col ^ (((row >> 2) & 1) << 3) : col;
}

// S^T copy for the readout: tile (fb, jb) -> rows 16 jb + li, columns
// 16 fb + 4 g .. +3 of sST.
template <typename F, typename T>
__device__ __forceinline__ void publish_state(const f32x4 *S, T *sST, int w,
                                              int g, int li) {
#pragma unroll
  for (int m = 0; m < F::FPW; ++m) {
#pragma unroll
    for (int mj = 0; mj < F::JPW; ++mj) {
      const int fb = tile_fb<F>(w, m), jb = tile_jb<F>(w, mj);
      const f32x4 s = S[m * F::JPW + mj];
      store4(sST + (16 * jb + li) * F::LQ + sst_col<T>(li, 16 * fb + 4 * g),
             s[0], s[1], s[2], s[3]);
    }
  }
}

// Exchange of segment aggregates between the workgroups of one (batch, head)
// unit, through that unit's line of the synchronisation area (see
// la_internal.h).  Only causal launches exchange inside the kernel, and
// every workgroup a wait depends on is running: segment indices follow
// start order.
//
// The XCDs of an MI355X do not share their L2 caches.  Each segment records
// the XCD it runs on in its unit's line when it starts.  A writer that finds
// every segment of its unit recorded on its own XCD stores its aggregate
// with plain stores, which land in that XCD's L2 (the L1 caches write
// through); otherwise with agent-scope stores, which write through to the
// device's coherence point.  The flag always goes to the coherence point,
// and its value says which: 2 for this XCD's L2, 1 for the coherence point.
// A reader polls the flags it needs at agent scope; once all are set it
// invalidates its L1, and also its L2 when any writer wrote through (so no
// stale line of an earlier launch hides that data), then reads the
// aggregates with plain loads.  A writer uses its L2 only when every
// segment of its unit, so every reader of it, runs on its XCD.
//
// Publishing: every wave waits until its aggregate stores have completed,
// then flag s is set.  The waits are bounded (a few seconds by default): if
// the area were ever corrupt they set the status word, poison the outputs
// that depend on the missing aggregates with NaN, and let the kernel finish
// instead of hanging.  At its very end every workgroup counts itself done;
// the last one clears the unit's line (flags, ticket, count, XCD records),
// so the area is zero again for the next launch.
__device__ __forceinline__ void store_agent(float *p, const f32x4 &v) {
  typedef unsigned long long u64;
  __hip_atomic_store(reinterpret_cast<u64 *>(p),
                     __builtin_bit_cast(u64, __builtin_shufflevector(v, v, 0, 1)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(reinterpret_cast<u64 *>(p) + 1,
                     __builtin_bit_cast(u64, __builtin_shufflevector(v, v, 2, 3)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The XCD this workgroup runs on as a 4-bit record, 1 + its id (hardware
// register XCC_ID, bits 0..3); 15 stands for "unknown" and never matches.
__device__ __forceinline__ unsigned xcc_record() {
  const unsigned x = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 0xfu;
  return x < 14 ? x + 1 : 15;
}

// Nibbles [0, n) of the record pair (r0: segments 0..7, r1: 8..15) all
// equal to v.
__device__ __forceinline__ bool records_match(unsigned r0, unsigned r1, int n,
                                              unsigned v) {
  const int n0 = n < 8 ? n : 8, n1 = n > 8 ? n - 8 : 0;
  const unsigned m0 = n0 == 8 ? ~0u : (1u << (4 * n0)) - 1u;
  const unsigned m1 = n1 == 8 ? ~0u : (1u << (4 * n1)) - 1u;
  const unsigned rep = v * 0x11111111u;
  return ((r0 ^ rep) & m0) == 0u && ((r1 ^ rep) & m1) == 0u;
}

__device__ __forceinline__ void publish_flag(unsigned *line, int seg,
                                             bool local) {
  // Each wave waits until its own aggregate stores have completed (a
  // workgroup barrier does not wait for them); only then is the flag set.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(line + seg, local ? 2u : 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Flags [0, need) of the line all set; call from every thread.  The wait
// polls at most spin_limit times; if it gives up, the status word gets
// kSyncStatusTimeout and the function returns true in every thread (the
// caller then poisons the outputs that depend on the missing aggregates).
__device__ __forceinline__ bool wait_flags(unsigned *line, int need,
                                           unsigned *status_word,
                                           unsigned spin_limit, int *sflag) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    unsigned spins = 0, f = 1u;
    bool gave_up = false;
    for (;;) {
      f = lane < need ? __hip_atomic_load(line + lane, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 2u;
      if (__all(f != 0u)) break;
      if (++spins > spin_limit) {
        gave_up = true;
        if (lane == 0)
          __hip_atomic_fetch_or(status_word, kSyncStatusTimeout,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (__any(f != 2u))
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    else
      asm volatile("buffer_inv sc0" ::: "memory");  // this CU's L1
    if (lane == 0) *sflag = gave_up ? 1 : 0;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*sflag) != 0;
}

__device__ __forceinline__ void count_done(unsigned *line, int nseg) {
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(line + kSyncDoneWord, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) ==
          static_cast<unsigned>(nseg - 1)) {
    for (int s = 0; s < nseg; ++s)
      __hip_atomic_store(line + s, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 0; i < 2; ++i)
      __hip_atomic_store(line + kSyncXccWord + i, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(line + kSyncTicketWord, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(line + kSyncDoneWord, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// RES: resident keys (causal, several segments, each at most KRES chunks):
// every segment, the last one included, runs phase 1 and keeps phi(K) of
// chunk c in slot c of sK for phase 2.
// SPLIT (non-causal, several segments): 0 = one launch with the exchange
// above; 1 = phase 1 only, the aggregate stored to its slot; 2 = phase 2
// only, reading every aggregate a launch with SPLIT = 1 stored before it on
// the same stream (the launch boundary orders them: no flags, no waits, no
// co-residency).
// DK: the decay mode of FwdShape (0 none, 1 per head, 2 per position).
template <typename T, int D, int DF, bool CAUSAL, bool MULTI, int DK,
          int MAP, bool RES = false, int SPLIT = 0, int VS = 1>
__global__ __launch_bounds__(kThreads,
                             (FwdShape<T, D, DF, DK, MAP>::WAVES_PER_SIMD))
void la_fwd_kernel(FwdArgs a) {
  using F = FwdShape<T, D, DF, DK, MAP>;
  constexpr bool DECAY = F::DECAY, SEL = F::SEL, WKEYS = F::WKEYS,
                 RW = F::RW;
  static_assert(!RES || (F::KRES > 0 && CAUSAL && MULTI), "resident keys");
  static_assert(SPLIT == 0 || (MULTI && !CAUSAL && !RES), "split launches");
  // the in-kernel exchange through the synchronisation area
  constexpr bool EXCH = MULTI && SPLIT == 0;
  constexpr bool ELU = MAP == kMapElu, PF = F::PF;
  constexpr int QW = F::QW, LX = F::LX;
  constexpr int C = F::C, LQ = F::LQ, LV = F::LV, DFP = F::DFP;
  constexpr int STRIPS = F::STRIPS, NJ = F::NJ, WPS = F::WPS;
  constexpr int NB1 = F::NB1, NB2 = F::NB2, TW = F::FPW * F::JPW;
  extern __shared__ __align__(16) unsigned char smem[];
  // NBUF sets of sQ, sKw, sV and sST; KS slots of sK (resident keys, or
  // one per set)
  T *sQ = reinterpret_cast<T *>(smem);
  T *sK = sQ + F::NBUF * F::SQ;
  T *sKw = WKEYS ? sK + F::SQ * F::KS : sK;
  T *sV = sK + F::SQ * F::KS + F::NBUF * F::SKW;
  T *sST = sV + F::NBUF * F::SV;
  T *sXq = sST + F::NST * F::SST;  // raw q, k rows (fused Performer)
  T *sXk = sXq + F::SX;
  float *gp = reinterpret_cast<float *>(sXk + F::SX);
  // fused Performer: the exponent offsets of the chunk's q rows, then of its
  // k rows (see stage_rows_pf), after the C + 8 + kMaxSegments words of gp:
  // the powers g^0 .. g^C, then the segment ticket, the two XCD record
  // words, the exchange's give-up flag and (per-position decay) the weights
  // of the segment aggregates
  float *pc0 = gp + C + 8 + kMaxSegments;
  float *sw = gp + C + 8;
  // per-position decay: the chunk tables, one per tile set (see sel_table)
  float *stab = pc0 + (PF ? 2 * C : 0);
  const float lsm = 0.5f * __builtin_log2f(static_cast<float>(DF));

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, li = lane & 15;
  // Workgroups are dispatched to the 8 XCDs round-robin by block index; the
  // segments of one unit are given blocks of one XCD (when the grid divides
  // evenly) so their exchange stays within one L2.
  int64_t blk = blockIdx.x;
  if (MULTI && a.nseg > 1 && gridDim.x % 8 == 0)
    blk = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  // With a value split (VS > 1) each (batch, head) unit is VS independent
  // computations over D of its VS D value columns: vunit numbers them (sync
  // line, aggregates), unit is the (batch, head) unit and part the columns.
  const int64_t vunit = blk / a.nseg;
  const int64_t unit = vunit / VS;
  const int part = static_cast<int>(vunit % VS);
  constexpr int LDV = D * VS;  // elements per row of v and out
  unsigned *line = EXCH && a.nseg > 1
                       ? a.sync + kSyncHeaderWords + vunit * kSyncLineWords
                       : nullptr;
  int seg = static_cast<int>(blk % a.nseg);
  // Causal segments take their index from the unit's ticket counter, in the
  // order they start: a segment then only ever waits for segments that are
  // already running, so no co-residency is needed.  The table of decay
  // powers and the constant tile parts are set up while the ticket is in
  // flight.
  const T *qb = static_cast<const T *>(a.q) + unit * a.n * QW;
  const T *kb = static_cast<const T *>(a.k) + unit * a.n * QW;
  const T *vb = static_cast<const T *>(a.v) + unit * a.n * LDV + part * D;
  // per-position decay: the unit's log decays [n]
  const float *lb = SEL ? a.log_decay + unit * a.n : nullptr;
  T *ob = static_cast<T *>(a.out) + unit * a.n * LDV + part * D;
  auto loadv = [&](Slab<T, D, C> &sv, int64_t r0, int rows) {
    if constexpr (VS > 1)
      sv.load_ld(vb, r0, rows, LDV, tid);
    else
      sv.load(vb, r0, rows, tid);
  };
  // Before the ticket returns, each workgroup loads the first phase-1 chunk
  // of the segment its block would take in block order (guess).  The
  // segments of a unit share an XCD, so together they bring every
  // segment's first chunk into that L2: a workgroup whose ticket differs
  // reloads from there.
  constexpr bool GUESS = EXCH && CAUSAL && F::NB1 == 1;
  const int guess = static_cast<int>(blk % a.nseg);
  Slab<T, QW, C> gk;
  Slab<T, D, C> gv;
  if (GUESS && a.nseg > 1) {
    const int64_t g0 = guess * a.seg_len;
    const int grows =
        static_cast<int>(max<int64_t>(0, min<int64_t>(C, a.n - g0)));
    gk.load(kb, g0 < a.n ? g0 : 0, grows, tid);
    loadv(gv, g0 < a.n ? g0 : 0, grows);
  }
  unsigned tk = 0u;
  if (EXCH && CAUSAL && a.nseg > 1 && tid == 0)
    tk = __hip_atomic_fetch_add(line + kSyncTicketWord, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
  const Decay dk(a.decay, static_cast<int>(unit % a.H));
  for (int i = tid; i <= C; i += kThreads) gp[i] = pow_int(dk.g, dk.lg, i);
  // Constant parts of the tiles: the ones block of sV (columns D, D + 4,
  // D + 8 and D + 12 = 1, the other 12 columns 0, every row) and, for
  // DF < 32, the zero k-padding columns of q', k' and S^T.  The four ones
  // columns give the state four equal copies of z, and the readout a
  // denominator in element 0 of every lane's accumulator (no cross-lane
  // step); nu is read from column D.
  for (int i = tid; i < F::NBUF * C * 16; i += kThreads)
    sV[(i / (C * 16)) * F::SV + ((i / 16) % C) * LV + D + i % 16] =
        from_f32<T>(i % 4 == 0 ? 1.f : 0.f);
  // Fused Performer: this wave's omega^T tiles times log2 e as A fragments,
  // rounded once to T and kept in registers (lane: feature 16 fb + li, d
  // values 32 kb + 8 g .. +7; for each d the 16 lanes read 16 consecutive
  // floats of omega [d][d_feat]).
  Frag<T> wf[PF ? F::TPW : 1][PF ? D / 32 : 1];
  if constexpr (PF) {
#pragma unroll
    for (int m = 0; m < F::TPW; ++m) {
      const int fb = F::NF >= kWaves ? w + kWaves * m : w % F::NF;
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          wf[m][kb].v[e] = from_f32<T>(
              a.omega[(32 * kb + 8 * g + e) * DF + 16 * fb + li] *
              1.4426950408889634f);
    }
  }
  if (DFP != DF) {
    // every slot of sQ, sK and sST (the padding is never written again)
    constexpr int NP = DFP - DF;
    for (int i = tid; i < (F::NBUF + F::KS) * C * NP; i += kThreads) {
      const int slot = i / (C * NP), row = (i / NP) % C, col = DF + i % NP;
      sQ[slot * F::SQ + row * LQ + col] = from_f32<T>(0.f);  // sK follows sQ
    }
    for (int i = tid; i < F::NST * (D + 16) * NP; i += kThreads) {
      const int row = (i / NP) % (D + 16);
      sST[(i / ((D + 16) * NP)) * F::SST + row * LQ +
          sst_col<T>(row, DF + i % NP)] = from_f32<T>(0.f);
    }
  }

  if (EXCH && CAUSAL && a.nseg > 1) {
    int *ticket = reinterpret_cast<int *>(gp + C + 1);
    if (tid == 0) {
      if (tk >= static_cast<unsigned>(a.nseg)) {  // corrupt area: in bounds
        __hip_atomic_fetch_or(a.sync + kSyncStatusWord, kSyncStatusCorrupt,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk %= static_cast<unsigned>(a.nseg);
      }
      *ticket = static_cast<int>(tk);
    }
    __syncthreads();
    seg = __builtin_amdgcn_readfirstlane(*ticket);
  }
  // this segment's XCD record (see the exchange above)
  const unsigned me = xcc_record();
  if (EXCH && a.nseg > 1 && tid == 0)
    __hip_atomic_fetch_or(line + kSyncXccWord + seg / 8, me << (4 * (seg % 8)),
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // wave 0, lanes 0 and 1: the unit's XCD records, read once every segment
  // has probably recorded (0 where not read)
  unsigned recs = 0u;

  const int64_t start = seg * a.seg_len;
  const int64_t end = min(a.n, start + a.seg_len);
  const int nch = static_cast<int>((end - start + C - 1) / C);
  // this workgroup writes the unit's final state (the last segment does)
  const bool keep_state = a.mu_out != nullptr && seg + 1 == a.nseg;
  // phi(K) of the whole segment stays in LDS from phase 1 to phase 2 (the
  // launch guarantees nch <= KRES)
  constexpr bool resident = RES;

  f32x4 S[TW];
  // per-position decay: sum of log2 gamma over this segment (phase 1)
  float seg_log2 = 0.f;
#pragma unroll
  for (int i = 0; i < TW; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunk helpers: valid rows of chunk c (0 past the end), the chunk whose
  // start a buffer resource for chunk c takes as its base (clamped to the
  // last one, so the base stays inside the array; padding chunks cover no
  // rows), and the tile set chunk c uses (c % 2 with two sets).
  const int last_rows =  // rows of the last chunk (1 .. C when nch > 0)
      static_cast<int>(end - (start + static_cast<int64_t>(nch - 1) * C));
  auto rows_of = [&](int c) -> int {
    return c < nch - 1 ? C : c == nch - 1 ? last_rows : 0;
  };
  auto clamp_chunk = [&](int c) -> int {
    return c < nch ? c : max(nch - 1, 0);
  };
  auto set_of = [&](int c) -> int { return F::NBUF == 2 ? (c & 1) : 0; };

  // Phase-2 register ring, first revolution; in the segmented kernel these
  // loads are issued once the aggregate is published and overlap the wait.
  Slab<T, QW, C> rq[NB2], rk2[NB2];
  Slab<T, D, C> rv2[NB2];
  LamSlab<C> rl2[NB2];
  auto load2 = [&](int c, Slab<T, QW, C> &sq, Slab<T, QW, C> &sk,
                   Slab<T, D, C> &sv, LamSlab<C> &sl) {
    const int64_t r0 = start + clamp_chunk(c) * C;
    const int rows = rows_of(c);  // 0 for padding chunks: zeros, no traffic
    sq.load(qb, r0, rows, tid);
    if (CAUSAL) {
      if (!resident) sk.load(kb, r0, rows, tid);
      loadv(sv, r0, rows);
      if constexpr (SEL) sl.load(lb, r0, rows, tid);
    }
  };
  auto ring2_first = [&]() {
#pragma unroll
    for (int b = 0; b < NB2; ++b) load2(b, rq[b], rk2[b], rv2[b], rl2[b]);
  };
  // Phase-2 staging of chunk c into its tile set (see the chunk loop).
  auto stage2 = [&](int c, const Slab<T, QW, C> &sq, const Slab<T, QW, C> &sk,
                    const Slab<T, D, C> &sv, const LamSlab<C> &sl) {
    const int sc = set_of(c);
    if constexpr (PF) {
      stage_rows_pf<T, D, C, LX>(sq, sXq, pc0, lsm, C, tid);
      if (CAUSAL)
        stage_rows_pf<T, D, C, LX>(sk, sXk, pc0 + C, lsm, rows_of(c), tid);
    } else {
      stage_queries<T, DF, C, LQ, ELU>(sq, sQ + sc * F::SQ, tid);
      if (CAUSAL && !resident)
        stage_keys<T, DF, C, LQ, WKEYS, true, ELU>(
            sk, sK + sc * F::SQ, sKw + sc * F::SQ, gp, dk.b, rows_of(c), tid);
    }
    if (CAUSAL) stage_values<T, D, C, LV>(sv, sV + sc * F::SV, tid);
    if constexpr (SEL)
      if (CAUSAL && w == 0) sel_table<C>(sl.v, stab + sc * F::TAB, lane);
    if constexpr (RW)
      if (CAUSAL && w == 0)
        rw_table<C>(stab + sc * F::TAB, gp, dk.b, rows_of(c), lane);
  };

  // The loops below run whole revolutions of their register ring (padding
  // chunks past nch have zero keys and store nothing) and stage chunk c + 1
  // while chunk c is multiplied.  With two tile sets (NBUF == 2) they do so
  // concurrently, with one barrier per chunk; with one set a barrier
  // separates the two.  The fused Performer map adds a step between staging
  // the raw rows and using the features.
  if constexpr (MULTI) {
    // ---------------- phase 1: segment aggregate from K, V ----------------
    // (not for the last causal segment, whose aggregate no other segment
    // needs, unless it keeps its keys resident)
    if (SPLIT != 2 && (!CAUSAL || seg + 1 < a.nseg || RES)) {
      Slab<T, QW, C> rk[NB1];
      Slab<T, D, C> rv[NB1];
      LamSlab<C> rl[NB1];
      auto load1 = [&](int c, Slab<T, QW, C> &sk, Slab<T, D, C> &sv,
                       LamSlab<C> &sl) {
        const int64_t r0 = start + clamp_chunk(c) * C;
        sk.load(kb, r0, rows_of(c), tid);
        loadv(sv, r0, rows_of(c));
        if constexpr (SEL) sl.load(lb, r0, rows_of(c), tid);
      };
#pragma unroll
      for (int b = 0; b < NB1; ++b) {
        if (GUESS && b == 0 && a.nseg > 1 && seg == guess) {
          rk[0] = gk;  // the guess was right
          rv[0] = gv;
          if constexpr (SEL) rl[0].load(lb, start, rows_of(0), tid);
        } else {
          load1(b, rk[b], rv[b], rl[b]);
        }
      }
      // phi(K) of chunk c: its resident slot (padding chunks: the unused
      // sQ), else the sK slot of its set
      auto keys1 = [&](int c) -> T * {
        if (resident)
          return c < nch ? sK + c * F::SQ : sQ + set_of(c) * F::SQ;
        return sK + set_of(c) * F::SQ;
      };
      auto stage1 = [&](int c, const Slab<T, QW, C> &sk,
                        const Slab<T, D, C> &sv, const LamSlab<C> &sl) {
        if constexpr (PF)
          stage_rows_pf<T, D, C, LX>(sk, sXk, pc0 + C, lsm, rows_of(c), tid);
        else
          stage_keys<T, DF, C, LQ, WKEYS, false, ELU>(
              sk, keys1(c), sKw + set_of(c) * F::SQ, gp, dk.b, rows_of(c),
              tid);
        stage_values<T, D, C, LV>(sv, sV + set_of(c) * F::SV, tid);
        if constexpr (SEL)
          if (w == 0) sel_table<C>(sl.v, stab + set_of(c) * F::TAB, lane);
        if constexpr (RW)
          if (w == 0)
            rw_table<C>(stab + set_of(c) * F::TAB, gp, dk.b, rows_of(c), lane);
      };
      auto features1 = [&](int c) {
        if constexpr (PF) {
          performer_features<F, T, false, true, WKEYS, false>(
              wf, sXq, sXk, pc0, pc0 + C, sQ, sK, sKw, gp, dk.b, rows_of(c),
              w, g, li);
          __syncthreads();
        }
      };
      __syncthreads();  // gp and the constant tile parts ready
      stage1(0, rk[0], rv[0], rl[0]);
      load1(NB1, rk[0], rv[0], rl[0]);
      if (EXCH && w == 0 && a.nseg > 1)
        recs = __hip_atomic_load(line + kSyncXccWord + (lane & 1),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      features1(0);
      for (int c0 = 0; c0 < nch; c0 += NB1) {
#pragma unroll
        for (int b = 0; b < NB1; ++b) {
          const int c = c0 + b, bn = (b + 1) % NB1;
          const int sc = F::NBUF == 2 && NB1 % 2 == 0 ? (b & 1) : set_of(c);
          const float *tabc = stab + sc * F::TAB;
          state_update<F>(S, WKEYS ? sKw + sc * F::SQ : keys1(c),
                          sV + sc * F::SV,
                          WKEYS || RW ? gp[rows_of(c)]
                          : SEL       ? tabc[3 * C]
                                      : 1.f,
                          w, g, li, ~0u, tabc + F::WOFF);
          if constexpr (SEL) seg_log2 += tabc[C - 1];
          if (F::NBUF == 1) __syncthreads();
          stage1(c + 1, rk[bn], rv[bn], rl[bn]);
          load1(c + 1 + NB1, rk[bn], rv[bn], rl[bn]);
          __syncthreads();
          features1(c + 1);
        }
      }
    }
    // With one segment the aggregate is already the state every row needs
    // (non-causal total).  With several, segment s combines the aggregates
    // A_j of the segments before it (causal) or of all segments
    // (non-causal): the state at position E is sum_j g^(E - end_j) A_j,
    // eqs 7-8 / 10-11 applied segment by segment, with E the segment start
    // (causal) or n.
    if (a.nseg > 1) {
      float *ub = a.states + vunit * a.nseg * static_cast<int64_t>(F::SLOT);
      const int need = CAUSAL ? seg : a.nseg;
      // the records as wave 0 read them, for every wave
      unsigned *srec = reinterpret_cast<unsigned *>(gp + C + 2);
      if (tid < 2) srec[tid] = recs;
      __syncthreads();
      const unsigned r0 = srec[0], r1 = srec[1];
      if (SPLIT == 1) {
        // aggregate-only launch: plain stores; the launch boundary makes
        // them visible to the readout launch that follows
        float *mine = ub + static_cast<int64_t>(seg) * F::SLOT;
#pragma unroll
        for (int m = 0; m < F::FPW; ++m)
#pragma unroll
          for (int mj = 0; mj < F::JPW; ++mj) {
            const int idx = tile_fb<F>(w, m) * F::NJA + tile_jb<F>(w, mj);
            *reinterpret_cast<f32x4 *>(mine + (idx * 64 + lane) * 4) =
                S[m * F::JPW + mj];
          }
        if (SEL && tid == 0) a.seg_log[vunit * a.nseg + seg] = seg_log2;
        return;
      }
      if (EXCH && (!CAUSAL || seg + 1 < a.nseg)) {
        // through this XCD's L2 when every segment of the unit runs on it
        const bool local = me < 15 && records_match(r0, r1, a.nseg, me);
        float *mine = ub + static_cast<int64_t>(seg) * F::SLOT;
#pragma unroll
        for (int m = 0; m < F::FPW; ++m)
#pragma unroll
          for (int mj = 0; mj < F::JPW; ++mj) {
            const int jb = tile_jb<F>(w, mj);
            const int idx = tile_fb<F>(w, m) * F::NJA + jb;
            float *dst = mine + (idx * 64 + lane) * 4;
            if (local)
              *reinterpret_cast<f32x4 *>(dst) = S[m * F::JPW + mj];
            else
              store_agent(dst, S[m * F::JPW + mj]);
          }
        if (SEL && tid == 0) {  // the segment's sum of log2 gamma, likewise
          float *dst = a.seg_log + vunit * a.nseg + seg;
          if (local)
            *dst = seg_log2;
          else
            __hip_atomic_store(dst, seg_log2, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        publish_flag(line, seg, local);
      }
      // the first chunk's phase-2 loads overlap the wait; the rest of the
      // ring follows the aggregates' loads, which would otherwise complete
      // only after them (loads complete in order)
      load2(0, rq[0], rk2[0], rv2[0], rl2[0]);
      // chunk 0 is staged while the predecessors finish (its tiles are free:
      // phase 1 ended with a workgroup barrier after its last use of them)
      stage2(0, rq[0], rk2[0], rv2[0], rl2[0]);
      bool gave_up = false;
      if (EXCH && need > 0)
        gave_up = wait_flags(line, need, a.sync + kSyncStatusWord,
                             a.spin_limit, reinterpret_cast<int *>(gp + C + 4));
      if constexpr (SEL) {
        // weight of aggregate j: the decay over the segments after it up
        // to this one, 2^(sum of their log2 gamma); wave 0 lane j takes
        // segment j and sums the totals after it
        static_assert(kMaxSegments <= kWave, "one segment per lane");
        if (w == 0) {
          const float tj =
              lane < need ? a.seg_log[vunit * a.nseg + lane] : 0.f;
          float suf = tj;  // inclusive suffix sum over lanes j .. need - 1
#pragma unroll
          for (int o = 1; o < kMaxSegments; o <<= 1) {
            const float y = __shfl_down(suf, o);
            if (lane + o < kMaxSegments) suf += y;
          }
          if (lane < need) sw[lane] = __builtin_amdgcn_exp2f(suf - tj);
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < TW; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int64_t epos = CAUSAL ? start : a.n;
      // Groups of GRP aggregates (about 12 tiles per lane, 24 with one
      // workgroup per CU), all loads of a group in flight together; members
      // past the last aggregate load nothing (a wave-uniform condition) and
      // add with weight 0.
      // With two tile sets, copies of the ones-block tile are not loaded:
      // their owners pass the sum on through tile set 1 of sQ (free until
      // chunk 1 is staged), read back after the next barrier.  Not with
      // padded features (d' < 32): the padding columns of sQ are zeroed
      // once per kernel and must stay zero.
      constexpr bool DEDUP = F::NBUF == 2 && F::NF < kWaves && DFP == DF;
      constexpr int TILES = F::OCC == 1 ? 24 : 12;
      constexpr int GRP = TW >= TILES ? 1 : pow2_floor(TILES / TW);
      for (int j0 = 0; j0 < need; j0 += GRP) {
        f32x4 buf[GRP][TW];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
          const int j = j0 + u;
          const float *sj = ub + static_cast<int64_t>(j) * F::SLOT;
#pragma unroll
          for (int m = 0; m < F::FPW; ++m)
#pragma unroll
            for (int mj = 0; mj < F::JPW; ++mj) {
              const int jb = tile_jb<F>(w, mj);
              const int idx = tile_fb<F>(w, m) * F::NJA + jb;
              buf[u][m * F::JPW + mj] =
                  j < need && !(DEDUP && dup_tile<F>(w, mj))
                      ? *reinterpret_cast<const f32x4 *>(
                            sj + (idx * 64 + lane) * 4)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
          const int j = j0 + u;
          const int64_t end_j = min(a.n, (j + 1) * a.seg_len);
          const float wj = j >= need ? 0.f
                           : SEL    ? sw[j]
                           : DECAY  ? pow_int(dk.g, dk.lg, epos - end_j)
                                    : 1.f;
#pragma unroll
          for (int i = 0; i < TW; ++i) S[i] += wj * buf[u][i];
        }
      }
      if (gave_up) {
        // a predecessor's aggregate never arrived: every output that
        // depends on it becomes NaN rather than silently wrong
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const float nan = __builtin_nanf("");
          S[i] = f32x4{nan, nan, nan, nan};
        }
      }
      if constexpr (DEDUP) {
        f32x4 *xs = reinterpret_cast<f32x4 *>(sQ + F::SQ);
#pragma unroll
        for (int mj = 0; mj < F::JPW; ++mj)
          if (owns_ones_tile<F>(w, mj))
            xs[tile_fb<F>(w, 0) * 64 + lane] = S[mj];
      }
#pragma unroll
      for (int b = 1; b < NB2; ++b) load2(b, rq[b], rk2[b], rv2[b], rl2[b]);
      load2(NB2, rq[0], rk2[0], rv2[0], rl2[0]);
    } else {
      ring2_first();
    }
  } else {
    ring2_first();
  }

  // ---------------- phase 2: chunk loop ----------------
  // Every wave runs the same instructions (masks instead of branches on its
  // output strip, apart from skipping whole key strips), so a chunk is one
  // straight block the compiler can interleave.  The fused Performer map
  // adds a feature step after each staging.
  auto features2 = [&](int c) {
    if constexpr (PF) {
      performer_features<F, T, true, CAUSAL, WKEYS, true>(
          wf, sXq, sXk, pc0, pc0 + C, sQ, sK, sKw, gp, dk.b, rows_of(c), w, g,
          li);
      __syncthreads();
    }
  };
  __syncthreads();  // gp and the constant tile parts ready, phase 1 done
  if constexpr (MULTI && F::NBUF == 2 && F::NF < kWaves && DFP == DF) {
    if (a.nseg > 1) {  // copies of the ones-block tile from their owners
      const f32x4 *xs = reinterpret_cast<const f32x4 *>(sQ + F::SQ);
#pragma unroll
      for (int mj = 0; mj < F::JPW; ++mj)
        if (dup_tile<F>(w, mj)) S[mj] = xs[tile_fb<F>(w, 0) * 64 + lane];
    }
  }
  publish_state<F>(S, sST, w, g, li);  // the entering state, set 0
  if (!(MULTI && a.nseg > 1)) {  // else staged during the exchange
    stage2(0, rq[0], rk2[0], rv2[0], rl2[0]);
    load2(NB2, rq[0], rk2[0], rv2[0], rl2[0]);
  }
  __syncthreads();
  features2(0);

  // This wave's output strip: the order alternates between groups of
  // STRIPS waves, so the two waves a SIMD usually holds (w, w + 4) take
  // strips of unequal causal work (k and STRIPS - 1 - k).
  const int tb =
      (w / STRIPS) % 2 == 0 ? w % STRIPS : STRIPS - 1 - w % STRIPS;
  const int jh = w / STRIPS;    // and its share of the column blocks
  const int t = 16 * tb + li;   // the output row this lane normalises
  // the entering state's weight in row t (per-position decay: per chunk)
  float gt = CAUSAL && !SEL ? gp[t + 1] : 1.f;
  // Causal mask of each P^T fragment pair kp: element e is key
  // s = 16 (2 kp + e / 4) + 4 g + e % 4, kept when s <= t.
  constexpr int NPK = (STRIPS + 1) / 2;
  u32x4 pm[NPK];
#pragma unroll
  for (int kp = 0; kp < NPK; ++kp) {
    pm[kp] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 16 * (2 * kp + e / 4) + 4 * g + e % 4;
      if (s <= t) pm[kp][e / 2] |= 0xffffu << (16 * (e % 2));
    }
  }
  // Decay weights b g^(t-s) of this lane's P^T elements (zero for s > t),
  // computed once where the registers allow (one workgroup per CU), else
  // per chunk from the table.
  constexpr bool PREW = (WKEYS || RW) && F::OCC == 1;
  float dw[PREW ? 4 * STRIPS : 1];
  if constexpr (PREW) {
#pragma unroll
    for (int sb = 0; sb < STRIPS; ++sb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int s = 16 * sb + 4 * g + rr;
        dw[4 * sb + rr] = s <= t ? dk.b * gp[t - s] : 0.f;
      }
  }
  constexpr int NJW = (NJ + WPS - 1) / WPS;
  // V^T fragment of the ones block (columns D + 4 k are 1 at every row, the
  // others 0): a constant, so it is never read from LDS
  const Frag<T> onesf = ones_frag<T>(li);
  for (int c0 = 0; c0 < nch; c0 += NB2) {
#pragma unroll
    for (int b = 0; b < NB2; ++b) {
      const int c = c0 + b, bn = (b + 1) % NB2;
      const int sc = F::NBUF == 2 && NB2 % 2 == 0 ? (b & 1) : set_of(c);
      const int sn = F::NBUF == 2 ? sc ^ 1 : 0;
      const int rows = rows_of(c);
      const T *sQc = sQ + sc * F::SQ;
      // resident keys: chunk c's phi(K) in slot c (padding chunks read a
      // stale slot; their outputs are dropped and their keys masked below)
      const T *sKc = resident ? sK + min(c, F::KS - 1) * F::SQ
                              : sK + sc * F::SQ;
      const T *sKwc = sKw + sc * F::SQ;
      const T *sVc = sV + sc * F::SV;
      const T *sSTc = CAUSAL && F::NST == 2 ? sST + sc * F::SST : sST;
      // per-position decay: this chunk's table, and row t's log2 decay
      const float *tabc = stab + sc * F::TAB;
      float Lt = 0.f;
      if constexpr (SEL) {
        if (CAUSAL) {
          Lt = tabc[t];
          gt = __builtin_amdgcn_exp2f(Lt);
        }
      }

      // ---- readout of strip tb: q' fragments, reused by every product ----
      Frag<T> qf[DFP / 32];
#pragma unroll
      for (int kq = 0; kq < DFP / 32; ++kq)
        load_frag8(qf[kq], sQc + t * LQ + 32 * kq + 8 * g);
      Frag<T> pf[NPK];
      // Key strips above the diagonal strip only hold masked products: they
      // are skipped (a branch on the wave's strip) from d' = 128 on, and at
      // d' = 64 unless the keys are resident; otherwise computed and masked
      // (no branch).  Measured: with resident keys, whose chunk loop has the
      // least other work, the branch costs more than the products it saves.
      constexpr bool SKIP = DFP >= 128 || (DFP >= 64 && !RES);
      if constexpr (CAUSAL) {
        f32x4 pt[STRIPS];
#pragma unroll
        for (int sb = 0; sb < STRIPS; ++sb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (!SKIP || sb <= tb) {
#pragma unroll
            for (int kq = 0; kq < DFP / 32; ++kq) {
              Frag<T> fa;
              load_frag8(fa, sKc + (16 * sb + li) * LQ + 32 * kq + 8 * g);
              acc = mma(fa, qf[kq], acc);
            }
          }
          // acc[rr] = q'_t . k'_s with s = 16 sb + 4 g + rr; with decay the
          // weights b g^(t-s), zero above the diagonal, are applied here,
          // without it the causal mask is applied to the packed pairs
          if constexpr (SEL) {
            // (1 - gamma_s) 2^(L_t - L_s) from this chunk's table
            const f32x4 ls =
                *reinterpret_cast<const f32x4 *>(tabc + 16 * sb + 4 * g);
            const f32x4 bs =
                *reinterpret_cast<const f32x4 *>(tabc + C + 16 * sb + 4 * g);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int s = 16 * sb + 4 * g + rr;
              // (above the diagonal the weight may overflow; the select
              // drops it)
              const float wgt = bs[rr] * __builtin_amdgcn_exp2f(Lt - ls[rr]);
              acc[rr] = s <= t ? acc[rr] * wgt : 0.f;
            }
          } else if (DECAY) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int s = 16 * sb + 4 * g + rr;
              if (PREW) acc[rr] *= dw[4 * sb + rr];
              else acc[rr] = s <= t ? acc[rr] * (dk.b * gp[s <= t ? t - s : 0])
                                    : 0.f;
            }
          }
          pt[sb] = acc;
        }
#pragma unroll
        for (int kp = 0; kp < NPK; ++kp) {
          frag_from_acc(pf[kp], pt[2 * kp],
                        2 * kp + 1 < STRIPS ? pt[2 * kp + 1]
                                            : f32x4{0.f, 0.f, 0.f, 0.f});
          if (!DECAY) frag_mask(pf[kp], pm[kp]);
        }
      }
      // This wave's column blocks: vblock(jj) = jh + WPS jj for jj < NJW,
      // then the ones block NJ (index NJW); their V^T fragments (split
      // assignment) are loaded once and, where the wave's state tiles are
      // the same blocks (SHARE), also serve the state update.
      auto vblock = [&](int jj) {
        return jj < NJW ? min(jh + WPS * jj, NJ) : NJ;
      };
      constexpr bool SHARE = CAUSAL && F::NF == STRIPS && F::NF < kWaves;
      Frag<T> vf[SHARE ? NJW + 1 : 1][NPK];
      if constexpr (SHARE) {
#pragma unroll
        for (int jj = 0; jj <= NJW; ++jj)
#pragma unroll
          for (int kp = 0; kp < NPK; ++kp) {
            if (jj == NJW)
              vf[jj][kp] = onesf;
            else
              load_frag_tr44(vf[jj][kp], sVc, LV, 32 * kp, 16 * vblock(jj),
                             g, li);
          }
      }
      // column block vblock(jj) of num^T = V^T P^T + g^(t+1) S^T Q'^T (the
      // ones block: its rows 0, 4, 8, 12 are the denominator,
      // sum_s P[t][s] + g^(t+1) q'_t . z, from the same rounded P and S copy
      // as the numerators)
      auto block = [&](int jj) {
        const int jb = vblock(jj);
        // without decay g^(t+1) = 1: both products share one accumulator
        f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
        f32x4 &acc_i = DECAY ? ai : an;
        if constexpr (SHARE) {
#pragma unroll
          for (int kp = 0; kp < NPK; ++kp) an = mma(vf[jj][kp], pf[kp], an);
        } else if constexpr (CAUSAL) {
#pragma unroll
          for (int kp = 0; kp < NPK; ++kp) {
            if (!SKIP || 2 * kp <= tb) {  // pairs above it are zero
              Frag<T> fa = onesf;
              if (jj < NJW)
                load_frag_tr44(fa, sVc, LV, 32 * kp, 16 * jb, g, li);
              an = mma(fa, pf[kp], an);
            }
          }
        }
#pragma unroll
        for (int kq = 0; kq < DFP / 32; ++kq) {
          Frag<T> fa;
          load_frag8(fa, sSTc + (16 * jb + li) * LQ +
                             sst_col<T>(li, 32 * kq + 8 * g));
          acc_i = mma(fa, qf[kq], acc_i);
        }
        return DECAY ? an + gt * ai : an;
      };
      // the denominator of row t is element 0 of this lane's ones-block
      // accumulator (row 4 g of the tile); its reciprocal (hardware, within
      // 1 ulp) scales the numerators
      const float den = block(NJW)[0];
      const float rden = __builtin_amdgcn_rcpf(den);
      // training forward: each row's denominator, for the backward pass
      // (the waves with jh == 0 hold every row of their strip once)
      if (a.den_out && part == 0 && jh == 0 && g == 0 && t < rows)
        a.den_out[unit * a.n + start + clamp_chunk(c) * C + t] = den;
      // the chunk's output rows (none for padding chunks); stores of rows
      // past the end and of blocks past the last are dropped
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc(ob + (start + clamp_chunk(c) * C) * LDV,
                    rows > 0 ? static_cast<unsigned>((rows - 1) * LDV + D) *
                                   sizeof(T)
                             : 0u);
#pragma unroll
      for (int jj = 0; jj < NJW; ++jj) {
        const f32x4 o = block(jj) * rden;
        // o[rr]: column j = 16 jb + 4 g + rr of output row t
        const int jb = jh + WPS * jj;
        const unsigned off = NJ % WPS == 0 || jb < NJ
                                 ? (t * LDV + 16 * jb + 4 * g) * sizeof(T)
                                 : kNoAccess;
        buffer_store4(ro, off, o[0], o[1], o[2], o[3], T{});
      }
      // the output stores issue here, before any wait for the next chunk's
      // loads that the staging below needs (measured faster except with
      // the fused Performer map, whose loop is scheduled better without)
      if constexpr (!PF) __builtin_amdgcn_sched_barrier(0);

      if constexpr (CAUSAL) {
        // ---- state update: S <- g^r S + (w.K')^T [V | 1] ----
        // (also after the last chunk, where the state only matters when it
        // is handed out, and on padding chunks, whose keys are zero)
        const T *sKu = WKEYS ? sKwc : sKc;
        const float gr = WKEYS || RW ? gp[rows] : SEL ? tabc[3 * C] : 1.f;
        const unsigned kmask = RES && c >= nch ? 0u : ~0u;
        if constexpr (SHARE) {
          // tile (w % NF, tile_jb(w, m)) uses column block vblock(m)
          static_assert(F::FPW == 1 && F::JPW <= NJW + 1, "tile layout");
          Frag<T> af[NPK];
#pragma unroll
          for (int kp = 0; kp < NPK; ++kp) {
            load_frag_tr44(af[kp], sKu, LQ, 32 * kp, 16 * tile_fb<F>(w, 0), g,
                           li);
            if (RES) frag_mask(af[kp], u32x4{kmask, kmask, kmask, kmask});
            if constexpr (SEL || RW)  // positions 32 kp + 4 g + e, then + 16
              frag_scale(af[kp],
                         *reinterpret_cast<const f32x4 *>(tabc + F::WOFF +
                                                          32 * kp + 4 * g),
                         *reinterpret_cast<const f32x4 *>(
                             tabc + F::WOFF + 32 * kp + 16 + 4 * g));
          }
#pragma unroll
          for (int m = 0; m < F::JPW; ++m) {
            f32x4 acc = S[m] * gr;
#pragma unroll
            for (int kp = 0; kp < NPK; ++kp) acc = mma(af[kp], vf[m][kp], acc);
            S[m] = acc;
          }
        } else {
          state_update<F>(S, sKu, sVc, gr, w, g, li, kmask, tabc + F::WOFF);
        }
      }
      if (F::NBUF == 1) __syncthreads();  // the one tile set is free again
      // ---- chunk c + 1 into its set; its ring slot reloaded ----
      stage2(c + 1, rq[bn], rk2[bn], rv2[bn], rl2[bn]);
      load2(c + 1 + NB2, rq[bn], rk2[bn], rv2[bn], rl2[bn]);
      if constexpr (F::NBUF == 2 && F::NST == 1) {
        // one S^T copy: every wave has read it for chunk c before the state
        // after chunk c replaces it
        if (CAUSAL) {
          __syncthreads();
          publish_state<F>(S, sST, w, g, li);
        }
      } else {
        if (CAUSAL) publish_state<F>(S, sST + sn * F::SST, w, g, li);
      }
      __syncthreads();
      features2(c + 1);
    }
  }

  // The state after the unit's last position (causal: after the last chunk's
  // update; non-causal: the total every row read), mu [d'][d] and nu [d'] in
  // fp32: tile (fb, jb) holds rows 16 fb + 4 g + r of columns 16 jb + li,
  // and the ones block's column 0 is nu.
  if (keep_state) {
    float *mu = a.mu_out + unit * static_cast<int64_t>(DF) * LDV + part * D;
    float *nu = a.nu_out + unit * static_cast<int64_t>(DF);
#pragma unroll
    for (int m = 0; m < F::FPW; ++m)
#pragma unroll
      for (int mj = 0; mj < F::JPW; ++mj) {
        const int fb = tile_fb<F>(w, m), jb = tile_jb<F>(w, mj);
        const f32x4 v = S[m * F::JPW + mj];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * fb + 4 * g + r;
          if (jb < NJ) mu[static_cast<int64_t>(f) * LDV + 16 * jb + li] = v[r];
          else if (jb == NJ && li == 0 && part == 0) nu[f] = v[r];
        }
      }
  }
  if (EXCH && a.nseg > 1) count_done(line, a.nseg);
}

}  // namespace la
