// Gradients of the causal forward (training), on gfx950 matrix cores.
//
// The forward reads out out_t = num_t / den_t with num_t = q'_t mu_t and
// den_t = q'_t . nu_t ("2.2 Linear Attention" eqs 7-11).  For a gradient
// dout of the outputs, let
//   G_t  = [dout_t / den_t | -(dout_t . out_t) / den_t]   (d + 1 values)
//   V+_s = [v_s | 1],   w_ts = b g^(t-s) for s <= t  (g = b = 1 without decay)
// (G's last value is carried as a bf16 pair hi + lo, matched by two ones in
// V+, and formed from the rounded dout / den, so that G_t . V+_s cancels
// to fp32 precision where the exact sum does: for one position, out = v and
// the gradients of q and k are exactly zero.)
// Differentiating the recurrence (the oracle's adjoint, regrouped) gives
// three unnormalised causal linear attentions:
//   dq'_t = sum_{s<=t} w_ts (G_t . V+_s) k'_s    query G,  key V+, value K'
//   dk'_s = sum_{t>=s} w_ts (G_t . V+_s) q'_t    query V+, key G,  value Q'
//   dv_s  = sum_{t>=s} w_ts (q'_t . k'_s) G_t    query K', key Q', value G
// the last two running backwards through the sequence; then dq = phi'(q)
// dq' and dk = phi'(k) dk' (elu + 1: 1 for x > 0, e^x else).
//
// Each of these is computed chunk by chunk exactly like the forward's
// numerator (C = 64 rows, local t, s, state S before the chunk):
//   out_t = sum_{s<=t} b g^(t-s) (X_t . Y_s) Z_s + g^(t+1) X_t S
//   S    <- g^r S + sum_s b g^(r-1-s) Y_s^T Z_s            (r valid rows)
// with (X, Y, Z) the (query, key, value) above; the reverse-order roles
// take the chunks from the last to the first and the rows of each chunk
// in reverse, so the same formulas read the sequence backwards.
//
// A preparation pass first writes, once per row, the operands every role
// shares: G~ (G padded to a multiple of 32 columns, its last value as the
// hi + lo pair), and for elu + 1 the features K' and Q'.  The role kernels
// then only copy tiles.
//
// Two kernels run the roles.  bf16 at d = 128 takes the segmented roles
// (see la_bwd_seg_kernel below): a workgroup per (role, unit, segment of the
// sequence) owns all output columns, with the segments' aggregates combined
// across two launches; dk and dv share one workgroup, since their states
// are transposes of each other.  Other sizes and fp32 take the column-block kernel:
// one 256-thread workgroup (4 waves) per (unit, role, block of 16 output
// columns), each walking its unit's whole sequence, all in one launch; the
// roles and blocks of a unit are independent, so no segment exchange is
// needed, but every workgroup recomputes the scores of its role, and the
// rows it shares with the unit's other workgroups come mostly from L2.
#include <algorithm>
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

namespace {

constexpr int kBThreads = 256;
constexpr int kBWaves = kBThreads / kWave;  // one 16-row output strip each
constexpr int kBC = 64;                     // chunk rows
constexpr int kRoleDQ = 0, kRoleDK = 1, kRoleDV = 2;

// LDS row stride (elements) for w elements: 16 mod 32 for bf16 (conflict-
// free transposing reads), +4 for fp32.
template <typename T>
constexpr int bstride(int w) {
  return sizeof(T) == 2 ? (w % 32 == 16 ? w : w + 16) : w + 4;
}

template <typename T, int D, int DF, int ROLE, bool DECAY, bool SEL = false>
struct BShape {
  // X and Y are G and V+ (d + 2 wide: the last value of G as a pair,
  // padded to a multiple of 32) for the dq and dk roles, and K', Q' (d'
  // wide, at least 32) for dv
  static constexpr bool GV = ROLE != kRoleDV;
  static constexpr int KX = GV ? (D + 2 + 31) / 32 * 32 : (DF < 32 ? 32 : DF);
  static constexpr int LX = bstride<T>(KX);
  static constexpr int LZ = bstride<T>(16);
  static constexpr int NT = KX / 16;                 // 16 x 16 state tiles
  static constexpr int TPW = (NT + kBWaves - 1) / kBWaves;
  static constexpr int SX = kBC * LX, SZ = kBC * LZ, SST = 16 * LX;
  // g^0 .. g^C, or with a decay per position the chunk's table (3 C + 4)
  static constexpr int TAB = SEL ? 3 * kBC + 4 : kBC + 4;
  static constexpr size_t lds_bytes =
      sizeof(T) * (SX * 2 + SZ + SST) + sizeof(float) * TAB;
};

// 16-byte pieces of a [C][W] row-major slab (consecutive threads take
// consecutive pieces) of rows row0 .. row0 + rows - 1 of a matrix whose
// rows are LD elements long, starting at column col0; rows past `rows`
// read zero (the buffer resource ends there).
template <typename T, int W, int LD, int NTH = kBThreads>
struct BSlab {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int PPR = W / VEC;
  static constexpr int PIECES = kBC * PPR;
  static constexpr int PER = (PIECES + NTH - 1) / NTH;
  static constexpr bool EXACT = PIECES % NTH == 0;
  static constexpr int THREADS = NTH;
  u32x4 v[PER];
  __device__ __forceinline__ void load(const T *base, int64_t row0, int rows,
                                       int col0, int tid) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(
        base + row0 * LD, static_cast<unsigned>(rows) * LD * sizeof(T));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + NTH * i;
      if (EXACT || p < PIECES)
        v[i] = buffer_load16(
            r, static_cast<unsigned>(((p / PPR) * LD + col0 +
                                      (p % PPR) * VEC) * sizeof(T)));
    }
  }
};

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float sum_group(float x) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// The values of one 16-byte piece as floats (8 bf16 or 4 fp32).
template <typename T>
__device__ __forceinline__ void piece_to_f32(const u32x4 &x,
                                             float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(x[i]);
      f[2 * i + 1] = bf16_hi(x[i]);
    }
  } else {
    const f32x4 y = __builtin_bit_cast(f32x4, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = y[i];
  }
}
template <typename T>
__device__ __forceinline__ u32x4 f32_to_piece(const float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                 pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
  } else {
    const f32x4 y = {f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(u32x4, y);
  }
}

__device__ __forceinline__ float phi(float x, bool elu) {
  return elu ? elu_plus_one(x) : x;
}
__device__ __forceinline__ float dphi(float x, bool elu) {  // d phi / d x
  return elu ? (x > 0.f ? 1.f : expf(x)) : 1.f;
}

// A decay per position (lam = log gamma, Mamba's input-dependent step):
// the chunk's table, computed by the 64 lanes of one wave, lane p holding
// lam of the position at processing index p (0 past the valid rows, which
// then keep the state: gamma = 1, 1 - gamma = 0).  With L the sums of
// log2 gamma over processing indices:
//   forward (dq): L_p inclusive (positions start .. p), so the entering
//     state reads out with 2^(L_t), key s scores b_s 2^(L_t - L_s) and
//     enters the state with b_s 2^(L_last - L_s);
//   reverse (dk, dv): L_p exclusive (the positions after p's, up to the
//     chunk's end), so the entering state reads out with b_t 2^(L_t), key
//     s scores b_t 2^(L_t - L_s) and enters with 2^(L_all - L_s): in the
//     adjoint the weight 1 - gamma belongs to the earlier position, which
//     is the query there.
// tab[p] = L_p, tab[C + p] = 1 - gamma_p, tab[2 C + p] = the state-update
// weight of key p (0 past the valid rows), tab[3 C] = 2^(sum of the chunk).
template <bool REV>
__device__ __forceinline__ float gate_table(float lam, float *tab, int lane,
                                            int rows) {
  constexpr int C = kBC;
  static_assert(C == kWave, "one row per lane");
  constexpr float kLog2e = 1.4426950408889634f;
  // below -104 exp(lam) is 0 in fp32; the floor keeps the sums finite for
  // lam = -inf (a full reset)
  lam = fmaxf(lam, -104.f);
  const float l = lam * kLog2e;
  float L = l;
#pragma unroll
  for (int o = 1; o < C; o <<= 1) {
    const float y = __shfl_up(L, o);
    if (lane >= o) L += y;
  }
  const float all = __shfl(L, C - 1);
  if (REV) L -= l;
  const float beta = -expm1f(lam);  // 1 - gamma, accurate near gamma = 1
  tab[lane] = L;
  tab[C + lane] = beta;
  tab[2 * C + lane] =
      lane < rows ? (REV ? 1.f : beta) * __builtin_amdgcn_exp2f(all - L) : 0.f;
  if (lane == 0) tab[3 * C] = __builtin_amdgcn_exp2f(all);
  return all;  // the chunk's sum of log2 gamma
}

// The table's uses: the causal weights of query t's scores against keys
// s = 16 sb + 4 g + rr (above the diagonal the power may overflow: the
// select drops it), the entering state's readout weight of query t, and
// the state-update weights of keys 32 kb + 8 g + e (lo) and + 4 (hi).
template <bool REV>
__device__ __forceinline__ void gate_scores(f32x4 &acc, const float *tab,
                                            int t, int sb, int g) {
  constexpr int C = kBC;
  const f32x4 ls = *reinterpret_cast<const f32x4 *>(tab + 16 * sb + 4 * g);
  const f32x4 bs = *reinterpret_cast<const f32x4 *>(tab + C + 16 * sb + 4 * g);
  const float lt = tab[t], bt = tab[C + t];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int s = 16 * sb + 4 * g + rr;
    const float wgt = (REV ? bt : bs[rr]) * __builtin_amdgcn_exp2f(lt - ls[rr]);
    acc[rr] = s <= t ? acc[rr] * wgt : 0.f;
  }
}
template <bool REV>
__device__ __forceinline__ float gate_readout(const float *tab, int t) {
  const float p = __builtin_amdgcn_exp2f(tab[t]);
  return REV ? tab[kBC + t] * p : p;
}
__device__ __forceinline__ void gate_update(const float *tab, int g,
                                            f32x4 (&wlo)[kBC / 32],
                                            f32x4 (&whi)[kBC / 32]) {
#pragma unroll
  for (int kb2 = 0; kb2 < kBC / 32; ++kb2) {
    wlo[kb2] = *reinterpret_cast<const f32x4 *>(tab + 2 * kBC + 32 * kb2 + 8 * g);
    whi[kb2] =
        *reinterpret_cast<const f32x4 *>(tab + 2 * kBC + 32 * kb2 + 8 * g + 4);
  }
}

// One role's workgroup: output columns 16 blk .. 16 blk + 15 of unit.  The
// dq and dk roles write feature gradients, d' wide (times phi' for elu + 1,
// where d' = d); with FG (the Performer map) they go to the workspace in
// fp32 (dqf, dkf) and a conversion pass takes them through the map.  SEL:
// a decay per position (a.lam) instead of one per head (DECAY is set too).
template <typename T, int D, int DF, int ROLE, bool DECAY, bool ELU,
          bool FG = false, bool SEL = false>
__device__ __forceinline__ void bwd_role(const BwdArgs &a, int64_t unit,
                                         int blk, unsigned char *smem) {
  static_assert(!SEL || DECAY, "a decay per position is a decay");
  using F = BShape<T, D, DF, ROLE, DECAY, SEL>;
  constexpr int C = kBC, KX = F::KX, LX = F::LX, LZ = F::LZ;
  constexpr bool GV = F::GV, REV = ROLE != kRoleDQ;
  constexpr int VEC = 16 / sizeof(T);
  T *sX = reinterpret_cast<T *>(smem);           // queries X
  T *sY = sX + F::SX;                            // keys Y
  T *sZ = sY + F::SX;                            // values Z (16 columns)
  T *sST = sZ + F::SZ;                           // S^T copy
  float *gp = reinterpret_cast<float *>(sST + F::SST);  // g^0 .. g^C
  float *tab = gp;  // SEL: the chunk's table (gate_table) instead

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int col0 = 16 * blk;
  const int h = static_cast<int>(unit % a.H);
  constexpr bool HD = DECAY && !SEL;  // one decay per head
  const float gdec = HD ? a.decay[h] : 1.f, bdec = HD ? 1.f - gdec : 1.f;
  const float lg = log2f(gdec);
  if constexpr (!SEL)
    for (int i = tid; i <= C; i += kBThreads) gp[i] = pow_int(gdec, lg, i);
  const float *lb = SEL ? a.lam + unit * a.n : nullptr;

  const int64_t n = a.n;
  const T *qb = static_cast<const T *>(a.q) + unit * n * D;
  const T *kb = static_cast<const T *>(a.k) + unit * n * D;
  const T *vb = static_cast<const T *>(a.v) + unit * n * D;
  constexpr int KG = backward_gwidth(D);  // G~ row width
  const T *gtb = static_cast<const T *>(a.gt) + unit * n * KG;
  const T *kfb = static_cast<const T *>(a.kf) + unit * n * DF;
  const T *qfb = static_cast<const T *>(a.qf) + unit * n * DF;
  // output rows: d' feature gradients (dq, dk) or d values (dv)
  constexpr int RW = ROLE == kRoleDV ? D : DF;
  using RT = std::conditional_t<FG && ROLE != kRoleDV, float, T>;
  void *rb = ROLE == kRoleDQ ? (FG ? a.dqf : a.dq)
             : ROLE == kRoleDK ? (FG ? a.dkf : a.dk)
                               : a.dv;
  RT *res = static_cast<RT *>(rb) + unit * n * RW;

  // Constant parts: the padding columns of X and Y past the data (zero for
  // every row; G~ rows are copied whole, the ones columns of V+ are written
  // per chunk).
  constexpr int XW = GV ? D + 2 : DF;  // written columns of X, Y
  for (int i = tid; i < C * (KX - XW); i += kBThreads) {
    const int row = i / (KX - XW), col = XW + i % (KX - XW);
    sX[row * LX + col] = from_f32<T>(0.f);
    sY[row * LX + col] = from_f32<T>(0.f);
  }

  const int nch = static_cast<int>((n + C - 1) / C);
  // Physical chunk of processing step c, its first row and valid rows.
  auto chunk_of = [&](int c) { return REV ? nch - 1 - c : c; };
  auto rows_of = [&](int c) -> int {
    if (c >= nch) return 0;
    const int64_t r0 = static_cast<int64_t>(chunk_of(c)) * C;
    return static_cast<int>(min<int64_t>(C, n - r0));
  };
  auto row0_of = [&](int c) -> int64_t {
    return c >= nch ? 0 : static_cast<int64_t>(chunk_of(c)) * C;
  };

  // Register ring (one chunk ahead).  GV roles: G~ and v full rows, the
  // K' block (dq) or Q' block (dk).  dv: K', Q' full rows, the G~ block.
  BSlab<T, KG, KG> rg;         // GV: G~
  BSlab<T, D, D> r1;           // GV: v
  BSlab<T, DF, DF> r1f, r2f;   // dv: K' (r1f), Q' (r2f)
  BSlab<T, 16, DF> rz;         // GV: K' or Q' block
  BSlab<T, 16, KG> rzg;        // dv: G~ block
  // SEL: lam of processing index `lane` of the chunk (wave 0; 0 past the
  // valid rows, which are out of the buffer resource)
  float laml = 0.f;
  auto load = [&](int c) {
    const int64_t r0 = row0_of(c);
    const int rows = rows_of(c);
    if constexpr (SEL) {
      if (w == 0) {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(lb + r0, static_cast<unsigned>(rows) * sizeof(float));
        const int rr = REV && lane < rows ? rows - 1 - lane : lane;
        laml = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       r, static_cast<unsigned>(rr) * 4u, 0, 0));
      }
    }
    if constexpr (GV) {
      rg.load(gtb, r0, rows, 0, tid);
      r1.load(vb, r0, rows, 0, tid);
      rz.load(ROLE == kRoleDQ ? kfb : qfb, r0, rows, col0, tid);
    } else {
      r1f.load(kfb, r0, rows, 0, tid);
      r2f.load(qfb, r0, rows, 0, tid);
      rzg.load(gtb, r0, rows, col0, tid);
    }
  };
  // Copy a slab's pieces into a tile of row stride L (rows in processing
  // order; pieces of rows past the end are zero).
  auto put = [&](const auto &sl, T *dst, int L, auto trow) {
    using S = std::remove_cv_t<std::remove_reference_t<decltype(sl)>>;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
      const int p = tid + S::THREADS * i;
      if (S::EXACT || p < S::PIECES)
        *reinterpret_cast<u32x4 *>(dst + trow(p / S::PPR) * L +
                                   (p % S::PPR) * VEC) = sl.v[i];
    }
  };

  // Staging of processing step c (rows in processing order: raw row r of a
  // reversed chunk goes to tile row rows - 1 - r; rows past the end are 0).
  auto stage = [&](int c) {
    const int rows = rows_of(c);
    auto trow = [&](int r) { return REV && r < rows ? rows - 1 - r : r; };
    if constexpr (SEL)
      if (w == 0) gate_table<REV>(laml, tab, lane, rows);
    if constexpr (GV) {
      // G~ as it is; V+ = [v | 1 | 1] (0 past the end)
      T *sG = ROLE == kRoleDQ ? sX : sY;
      T *sV = ROLE == kRoleDQ ? sY : sX;
      put(rg, sG, LX, trow);
      put(r1, sV, LX, trow);
      if (tid < C) {
        const int t = trow(tid);
        const T one = from_f32<T>(tid < rows ? 1.f : 0.f);
        sV[t * LX + D] = one;
        sV[t * LX + D + 1] = one;
      }
    } else {
      put(r1f, sX, LX, trow);
      put(r2f, sY, LX, trow);
    }
    if constexpr (GV)
      put(rz, sZ, LZ, trow);
    else
      put(rzg, sZ, LZ, trow);
  };

  // State tiles of this wave: S (features 16 fb .. +16, the 16 value
  // columns), fb = w + kBWaves m; past NT: unused (kept zero).
  f32x4 S[F::TPW];
#pragma unroll
  for (int m = 0; m < F::TPW; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto publish = [&]() {  // S^T copy: row = value column, columns = features
#pragma unroll
    for (int m = 0; m < F::TPW; ++m) {
      const int fb = w + kBWaves * m;
      if (fb < F::NT)
        store4(sST + li * LX + 16 * fb + 4 * g, S[m][0], S[m][1], S[m][2],
               S[m][3]);
    }
  };

  const int tb = w;                 // this wave's output strip
  const int t = 16 * tb + li;       // the query row this lane reads out
  // dq, dk (elu + 1): the raw q or k of this lane's four output elements
  // (row t of the chunk, columns col0 + 4 g ..) for phi', loaded with the
  // chunk's operands (pfn) and moved to pfc once that chunk is staged, so
  // the load is never waited for at the output
  static_assert(!ELU || DF == D, "elu + 1 keeps d' = d");
  constexpr bool PFI = GV && ELU;
  using PV = std::conditional_t<sizeof(T) == 2, u32x2, u32x4>;
  PV pfn{}, pfc{};
  auto load_phi = [&](int c) {
    if constexpr (PFI) {
      const int rows = rows_of(c);
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc((ROLE == kRoleDQ ? qb : kb) + row0_of(c) * D,
                    static_cast<unsigned>(rows) * D * sizeof(T));
      // rows at or past the end are out of the resource and read zero
      const int rr = REV && t < rows ? rows - 1 - t : t;
      const unsigned off =
          static_cast<unsigned>(rr * D + col0 + 4 * g) * sizeof(T);
      if constexpr (sizeof(T) == 2)
        pfn = __builtin_bit_cast(
            PV, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      else
        pfn = buffer_load16(r, off);
    }
  };
  load(0);
  load_phi(0);
  __syncthreads();                  // gp and the constant parts ready
  stage(0);
  pfc = pfn;
  load(1);
  load_phi(1);
  publish();
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int rows = rows_of(c);
    // the entering state's readout weight of query t
    const float gt = !SEL ? gp[t + 1]
                     : REV ? tab[C + t] * __builtin_amdgcn_exp2f(tab[t])
                           : __builtin_amdgcn_exp2f(tab[t]);
    // ---- readout of strip tb ----
    Frag<T> xf[KX / 32];
#pragma unroll
    for (int kq = 0; kq < KX / 32; ++kq)
      load_frag8(xf[kq], sX + t * LX + 32 * kq + 8 * g);
    f32x4 pt[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (sb <= tb) {
#pragma unroll
        for (int kq = 0; kq < KX / 32; ++kq) {
          Frag<T> fa;
          load_frag8(fa, sY + (16 * sb + li) * LX + 32 * kq + 8 * g);
          acc = mma(fa, xf[kq], acc);
        }
      }
      // acc[rr]: key s = 16 sb + 4 g + rr, query t; causal weights
      if constexpr (SEL) {
        const f32x4 ls =
            *reinterpret_cast<const f32x4 *>(tab + 16 * sb + 4 * g);
        const f32x4 bs =
            *reinterpret_cast<const f32x4 *>(tab + C + 16 * sb + 4 * g);
        const float lt = tab[t], bt = tab[C + t];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int s = 16 * sb + 4 * g + rr;
          // (above the diagonal the power may overflow: the select drops it)
          const float wgt =
              (REV ? bt : bs[rr]) * __builtin_amdgcn_exp2f(lt - ls[rr]);
          acc[rr] = s <= t ? acc[rr] * wgt : 0.f;
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int s = 16 * sb + 4 * g + rr;
          acc[rr] = s <= t ? acc[rr] * (DECAY ? bdec * gp[s <= t ? t - s : 0]
                                              : 1.f)
                           : 0.f;
        }
      }
      pt[sb] = acc;
    }
    f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      if (2 * kp <= tb) {
        Frag<T> pf, zf;
        frag_from_acc(pf, pt[2 * kp], pt[2 * kp + 1]);
        load_frag_tr44(zf, sZ, LZ, 32 * kp, 0, g, li);
        an = mma(zf, pf, an);
      }
    }
#pragma unroll
    for (int kq = 0; kq < KX / 32; ++kq) {
      Frag<T> fa;
      load_frag8(fa, sST + li * LX + 32 * kq + 8 * g);
      ai = mma(fa, xf[kq], ai);
    }
    const f32x4 o = an + gt * ai;
    // o[r]: value column 4 g + r of query row t; times phi' for dq, dk
    if (t < rows) {
      const int64_t row = row0_of(c) + (REV ? rows - 1 - t : t);
      // dq, dk: times phi'(x) of the same elements of q or k
      float xin[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (PFI) {
        if constexpr (sizeof(T) == 2) {
          xin[0] = bf16_lo(pfc[0]);
          xin[1] = bf16_hi(pfc[0]);
          xin[2] = bf16_lo(pfc[1]);
          xin[3] = bf16_hi(pfc[1]);
        } else {
          const f32x4 y = __builtin_bit_cast(f32x4, pfc);
#pragma unroll
          for (int r = 0; r < 4; ++r) xin[r] = y[r];
        }
      }
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[r] = PFI ? o[r] * dphi(xin[r], true) : o[r];
      store4(res + row * RW + col0 + 4 * g, x[0], x[1], x[2], x[3]);
    }
    // ---- state update: S <- g^r S + (w Y)^T Z, the weights w_s =
    // b g^(r-1-s) of positions 32 kb + 8 g + e applied in registers ----
    const float gr = SEL ? tab[3 * C] : gp[rows];
    f32x4 wlo[C / 32], whi[C / 32];
    if constexpr (SEL) {
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2) {
        wlo[kb2] = *reinterpret_cast<const f32x4 *>(tab + 2 * C + 32 * kb2 +
                                                    8 * g);
        whi[kb2] = *reinterpret_cast<const f32x4 *>(tab + 2 * C + 32 * kb2 +
                                                    8 * g + 4);
      }
    } else if constexpr (DECAY) {
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s0 = 32 * kb2 + 8 * g + e, s1 = s0 + 4;
          wlo[kb2][e] = s0 < rows ? bdec * gp[rows - 1 - s0] : 0.f;
          whi[kb2][e] = s1 < rows ? bdec * gp[rows - 1 - s1] : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < F::TPW; ++m) {
      const int fb = w + kBWaves * m;
      if (fb < F::NT) {
        f32x4 acc = S[m] * gr;
#pragma unroll
        for (int kb2 = 0; kb2 < C / 32; ++kb2) {
          Frag<T> af, bf;
          load_frag_tr8(af, sY, LX, 32 * kb2, 16 * fb, g, li);
          if constexpr (DECAY) frag_scale(af, wlo[kb2], whi[kb2]);
          load_frag_tr8(bf, sZ, LZ, 32 * kb2, 0, g, li);
          acc = mma(af, bf, acc);
        }
        S[m] = acc;
      }
    }
    __syncthreads();   // the tile set is free again
    stage(c + 1);
    pfc = pfn;
    load(c + 2);
    load_phi(c + 2);
    publish();
    __syncthreads();
  }
}

// Preparation pass: per row of every unit, G~ = [g | h hi | h lo | 0 ..]
// with g = dout / den rounded to the storage type and h = -(g . out) (the
// dot product of the rounded g, in fp32; hi its rounding, lo the rest), and
// for elu + 1 the features K' = phi(k), Q' = phi(q).  LPR consecutive
// threads take one row, one 16-byte piece each; the row's dot product is
// summed across them.  Grid-stride over groups of rows.
template <typename T, int D, bool ELU>
__global__ __launch_bounds__(kBThreads) void la_bwd_prep_kernel(
    BwdArgs a, int64_t rows_total) {
  constexpr int VEC = 16 / sizeof(T), LPR = D / VEC, KG = backward_gwidth(D);
  constexpr int NPAD = (KG - D) / VEC;  // pieces of a G~ row past g
  constexpr int RPB = kBThreads / LPR;  // rows per block and step
  static_assert(NPAD <= LPR, "pad pieces");
  const int tid = threadIdx.x, j = tid % LPR;
  const int64_t nsteps = (rows_total + RPB - 1) / RPB;
  for (int64_t st = blockIdx.x; st < nsteps; st += gridDim.x) {
    const int64_t row = st * RPB + tid / LPR;
    // a row's LPR threads are consecutive and aligned, so they stay or
    // leave together and the sums below never read a departed lane
    if (row >= rows_total) break;
    const int64_t off = row * D + j * VEC;
    const u32x4 dop =
        *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.dout) + off);
    const u32x4 oup =
        *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.out) + off);
    const float rden = 1.f / a.den[row];
    float go[VEC], oo[VEC];
    piece_to_f32<T>(dop, go);
    piece_to_f32<T>(oup, oo);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      go[e] = round_to<T>(go[e] * rden);
      dot += go[e] * oo[e];
    }
    dot = sum_group<LPR>(dot);
    T *gr = static_cast<T *>(a.gt) + row * KG;
    *reinterpret_cast<u32x4 *>(gr + j * VEC) = f32_to_piece<T>(go);
    if (j < NPAD) {
      const float hh = -dot;
      const float hi = round_to<T>(hh), lo = hh - hi;
      float pad[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) pad[e] = 0.f;
      if (j == 0) {
        pad[0] = hi;
        pad[1] = lo;
      }
      *reinterpret_cast<u32x4 *>(gr + D + j * VEC) = f32_to_piece<T>(pad);
    }
    if constexpr (ELU) {
      const u32x4 qp =
          *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + off);
      const u32x4 kp =
          *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.k) + off);
      float qx[VEC], kx[VEC];
      piece_to_f32<T>(qp, qx);
      piece_to_f32<T>(kp, kx);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        qx[e] = phi(qx[e], true);
        kx[e] = phi(kx[e], true);
      }
      *reinterpret_cast<u32x4 *>(static_cast<T *>(a.qf) + off) =
          f32_to_piece<T>(qx);
      *reinterpret_cast<u32x4 *>(static_cast<T *>(a.kf) + off) =
          f32_to_piece<T>(kx);
    }
  }
}

// ---------------------------------------------------------------------------
// Segmented roles (bf16, d = 128).  One 512-thread workgroup (8 waves) per
// (role, unit, segment of the role's processing order) owns all d output
// columns, so a chunk's scores are formed once per 16-row strip instead of
// once per 16-column block.  Two launches, like the forward's non-causal
// split: PHASE 1 writes each segment's aggregate (its end state from a zero
// state) to the workspace; PHASE 2 sums the aggregates of the segments
// before it, each weighted by the decay over the rows between, and runs the
// chunk loop from that state.  No workgroup waits for another.
// Wave w = 4 jh + tb reads out strip tb for column blocks 4 jh .. 4 jh + 3
// and owns the state of column block w (all its feature tiles).  seg_role
// runs dq (both launches) and the dk aggregates; seg_dkv below reads out dk
// and dv together, so the dv role has no workgroup of its own.
// ---------------------------------------------------------------------------
constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / kWave;
constexpr int kSegD = 128;                                   // d built
constexpr int kSegTiles = backward_gwidth(kSegD) / 16;       // NT, at most
constexpr int kSegSlot = kSWaves * kSegTiles * 256;          // floats

// A decay per position: each segment's sum of log2 gamma over its rows,
// written by the aggregates launch after all aggregates ([role][unit][seg]).
__device__ __forceinline__ float *seg_total(const BwdArgs &a, int64_t units,
                                            int role, int64_t unit, int seg) {
  return a.agg + 2 * units * a.nseg * static_cast<int64_t>(kSegSlot) +
         (role * units + unit) * a.nseg + seg;
}

template <typename T, int ROLE>
struct SShape {
  static_assert(ROLE == kRoleDQ || ROLE == kRoleDK, "dq, dk layouts");
  static constexpr int D = kSegD;
  // queries and keys G~ and V+: d + 2 values padded to a multiple of 32
  static constexpr int KX = backward_gwidth(D);
  static constexpr int LX = bstride<T>(KX);
  static constexpr int LZ = bstride<T>(D);
  static constexpr int NT = KX / 16;
  static constexpr int SX = kBC * LX, SZ = kBC * LZ, SST = D * LX;
  // dq also stages the raw q rows (phi'(q) of its outputs)
  static constexpr int SP = ROLE == kRoleDQ ? SZ : 0;
  // the powers g^0 .. g^C, or with a decay per position the chunk's table
  static constexpr int TAB = 3 * kBC + 4;
  static constexpr size_t lds_bytes =
      sizeof(T) * (2 * SX + SZ + SST + SP) + sizeof(float) * TAB;
  // the aggregates launch stages only Y and Z: two workgroups fit a CU
  static constexpr size_t lds_bytes_agg =
      sizeof(T) * (SX + SZ) + sizeof(float) * TAB;
  static_assert(D / 16 == kSWaves, "one state column block per wave");
};

template <typename T, int ROLE, bool DECAY, bool ELU, int PHASE,
          bool SEL = false>
__device__ __forceinline__ void seg_role(const BwdArgs &a, int64_t units,
                                         int64_t unit, int seg,
                                         unsigned char *smem) {
  const int nseg = a.nseg;
  float *agg = a.agg;
  using F = SShape<T, ROLE>;
  constexpr int D = F::D, C = kBC, KX = F::KX, LX = F::LX, LZ = F::LZ;
  constexpr int NT = F::NT, KG = backward_gwidth(D);
  static_assert(ROLE == kRoleDQ || (ROLE == kRoleDK && PHASE == 1),
                "seg_dkv reads out dk");
  constexpr bool REV = ROLE != kRoleDQ;
  // PHASE 2: X, Y, Z, S^T, raw q (dq) and the powers of g; PHASE 1 reads
  // no queries and publishes no S^T: Y, Z and the powers only
  T *sX = reinterpret_cast<T *>(smem);           // queries X
  T *sY = PHASE == 1 ? sX : sX + F::SX;          // keys Y
  T *sZ = sY + F::SX;                            // values Z (all d columns)
  T *sST = sZ + F::SZ;                           // S^T copy
  T *sP = sST + F::SST;                          // raw q rows (dq)
  float *gp = reinterpret_cast<float *>(PHASE == 1 ? sST : sP + F::SP);
  float *tab = gp;  // SEL: the chunk's table (gate_table) instead

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tb = w % 4, jh = w / 4;
  const int h = static_cast<int>(unit % a.H);
  constexpr bool HD = DECAY && !SEL;  // one decay per head
  const float gdec = HD ? a.decay[h] : 1.f, bdec = HD ? 1.f - gdec : 1.f;
  const float lg = log2f(gdec);
  if constexpr (!SEL)
    for (int i = tid; i <= C; i += kSThreads) gp[i] = pow_int(gdec, lg, i);
  const float *lb = SEL ? a.lam + unit * a.n : nullptr;
  float laml = 0.f;  // SEL, wave 0: lam of processing index `lane`
  float segl = 0.f;  // SEL, wave 0: the segment's sum of log2 gamma so far

  const int64_t n = a.n;
  const T *qb = static_cast<const T *>(a.q) + unit * n * D;
  const T *kb = static_cast<const T *>(a.k) + unit * n * D;
  const T *vb = static_cast<const T *>(a.v) + unit * n * D;
  const T *gtb = static_cast<const T *>(a.gt) + unit * n * KG;
  T *res = static_cast<T *>(a.dq) + unit * n * D;

  // the zero padding columns of X and Y (G~ rows are copied whole, the
  // ones columns of V+ are written per chunk)
  constexpr int XW = D + 2;
  for (int i = tid; i < C * (KX - XW); i += kSThreads) {
    const int row = i / (KX - XW), col = XW + i % (KX - XW);
    if (PHASE == 2) sX[row * LX + col] = from_f32<T>(0.f);
    sY[row * LX + col] = from_f32<T>(0.f);
  }

  // processing steps of this segment (step c is physical chunk c, or
  // nch - 1 - c for the reverse-order roles)
  const int nch = static_cast<int>((n + C - 1) / C);
  const int cps = (nch + nseg - 1) / nseg;
  const int cb = seg * cps, ce = min(nch, cb + cps);
  auto chunk_of = [&](int c) { return REV ? nch - 1 - c : c; };
  auto rows_of = [&](int c) -> int {
    if (c >= ce) return 0;
    const int64_t r0 = static_cast<int64_t>(chunk_of(c)) * C;
    return static_cast<int>(min<int64_t>(C, n - r0));
  };
  auto row0_of = [&](int c) -> int64_t {
    return c >= ce ? 0 : static_cast<int64_t>(chunk_of(c)) * C;
  };

  // Register ring (one chunk ahead).  X is not needed in PHASE 1.  K' and
  // Q' are mapped from the raw k and q rows while staging (each workgroup
  // stages a row once).
  using SG = BSlab<T, KG, KG, kSThreads>;   // G~ rows
  using SD = BSlab<T, D, D, kSThreads>;     // v, k or q rows
  SG rg;
  SD r1, r2, r3;
  // rg = G~ (X of dq, Y of dk), r1 = v (V+), r2 = K' (dq) or Q' (dk), r3 =
  // the raw q rows (dq's phi'(q), staged to sP)
  constexpr bool NEED_G = PHASE == 2 || ROLE == kRoleDK;
  constexpr bool NEED_R1 = PHASE == 2 || ROLE == kRoleDQ;
  constexpr bool PFI = ROLE == kRoleDQ && ELU && PHASE == 2;
  auto load = [&](int c) {
    const int64_t r0 = row0_of(c);
    const int rows = rows_of(c);
    if constexpr (NEED_G) rg.load(gtb, r0, rows, 0, tid);
    if constexpr (NEED_R1) r1.load(vb, r0, rows, 0, tid);
    r2.load(ROLE == kRoleDQ ? kb : qb, r0, rows, 0, tid);
    if constexpr (PFI) r3.load(qb, r0, rows, 0, tid);
    if constexpr (SEL) {
      if (w == 0) {  // rows past the end are out of the resource: lam 0
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(lb + r0, static_cast<unsigned>(rows) * sizeof(float));
        const int rr = REV && lane < rows ? rows - 1 - lane : lane;
        laml = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       r, static_cast<unsigned>(rr) * 4u, 0, 0));
      }
    }
  };
  // the same with phi applied (elu + 1 in fp32, rounded once; rows past the
  // end stay zero)
  auto put_phi = [&](const SD &sl, T *dst, int L, auto trow, int rows) {
#pragma unroll
    for (int i = 0; i < SD::PER; ++i) {
      const int p = tid + SD::THREADS * i;
      if (SD::EXACT || p < SD::PIECES) {
        const int r = p / SD::PPR;
        u32x4 y = sl.v[i];
        if constexpr (ELU) {
          float f[SD::VEC];
          piece_to_f32<T>(sl.v[i], f);
#pragma unroll
          for (int e = 0; e < SD::VEC; ++e)
            f[e] = r < rows ? elu_plus_one_fast(f[e]) : 0.f;
          y = f32_to_piece<T>(f);
        }
        *reinterpret_cast<u32x4 *>(dst + trow(r) * L + (p % SD::PPR) * SD::VEC) =
            y;
      }
    }
  };
  auto put = [&](const auto &sl, T *dst, int L, auto trow) {
    using S = std::remove_cv_t<std::remove_reference_t<decltype(sl)>>;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
      const int p = tid + S::THREADS * i;
      if (S::EXACT || p < S::PIECES)
        *reinterpret_cast<u32x4 *>(dst + trow(p / S::PPR) * L +
                                   (p % S::PPR) * S::VEC) = sl.v[i];
    }
  };
  auto stage = [&](int c) {
    const int rows = rows_of(c);
    auto trow = [&](int r) { return REV && r < rows ? rows - 1 - r : r; };
    T *sG = ROLE == kRoleDQ ? sX : sY;
    T *sV = ROLE == kRoleDQ ? sY : sX;
    if constexpr (SEL)
      if (w == 0) segl += gate_table<REV>(laml, tab, lane, rows);
    if constexpr (NEED_G) put(rg, sG, LX, trow);
    if constexpr (NEED_R1) {
      put(r1, sV, LX, trow);
      if (tid < C) {
        const int t = trow(tid);
        const T one = from_f32<T>(tid < rows ? 1.f : 0.f);
        sV[t * LX + D] = one;
        sV[t * LX + D + 1] = one;
      }
    }
    put_phi(r2, sZ, LZ, trow, rows);
    if constexpr (PFI) put(r3, sP, LZ, trow);
  };

  // this wave's state: column block w, feature tiles 0 .. NT - 1
  f32x4 S[NT];
#pragma unroll
  for (int fb = 0; fb < NT; ++fb) S[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto slot = [&](int sg) {
    return agg + ((static_cast<int64_t>(ROLE) * units + unit) * nseg +
                  sg) *
                     kSegSlot +
           (w * kSegTiles) * 256 + lane * 4;
  };
  if constexpr (PHASE == 2) {
    // the entering state: the aggregates before this segment, each carried
    // over the rows between it and this segment (whole chunks)
    // (SEL: carried over the segments between by their sums of log2 gamma)
    float between = 0.f;
    for (int i = 0; i < seg; ++i) {
      const int sg = SEL ? seg - 1 - i : i;
      const float wgt =
          SEL   ? __builtin_amdgcn_exp2f(between)
          : HD  ? pow_int(gdec, lg,
                          static_cast<int64_t>(seg - sg - 1) * cps * C)
                : 1.f;
      if constexpr (SEL) between += *seg_total(a, units, ROLE, unit, sg);
      const float *src = slot(sg);
#pragma unroll
      for (int fb = 0; fb < NT; ++fb)
        S[fb] += wgt * *reinterpret_cast<const f32x4 *>(src + fb * 256);
    }
  }
  auto publish = [&]() {  // S^T rows 16 w .. + 15 (this wave's columns)
#pragma unroll
    for (int fb = 0; fb < NT; ++fb)
      store4(sST + (16 * w + li) * LX + 16 * fb + 4 * g, S[fb][0], S[fb][1],
             S[fb][2], S[fb][3]);
  };
  auto state_update = [&](int c) {
    const int rows = rows_of(c);
    const float gr = SEL ? tab[3 * C] : gp[rows];
    f32x4 wlo[C / 32], whi[C / 32];
    if constexpr (SEL) {
      gate_update(tab, g, wlo, whi);
    } else if constexpr (DECAY) {
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s0 = 32 * kb2 + 8 * g + e, s1 = s0 + 4;
          wlo[kb2][e] = s0 < rows ? bdec * gp[rows - 1 - s0] : 0.f;
          whi[kb2][e] = s1 < rows ? bdec * gp[rows - 1 - s1] : 0.f;
        }
    }
    // the weights go on this wave's one Z block (positions along the
    // contraction, as in the Y fragments), not on its NT Y fragments
    Frag<T> bf[C / 32];
#pragma unroll
    for (int kb2 = 0; kb2 < C / 32; ++kb2) {
      load_frag_tr8(bf[kb2], sZ, LZ, 32 * kb2, 16 * w, g, li);
      if constexpr (DECAY) frag_scale(bf[kb2], wlo[kb2], whi[kb2]);
    }
#pragma unroll
    for (int fb = 0; fb < NT; ++fb) {
      f32x4 acc = S[fb] * gr;
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2) {
        Frag<T> af;
        load_frag_tr8(af, sY, LX, 32 * kb2, 16 * fb, g, li);
        acc = mma(af, bf[kb2], acc);
      }
      S[fb] = acc;
    }
  };

  const int t = 16 * tb + li;  // the query row this lane reads out

  load(cb);
  __syncthreads();  // gp and the constant parts ready
  stage(cb);
  load(cb + 1);
  if constexpr (PHASE == 2) publish();
  __syncthreads();

  for (int c = cb; c < ce; ++c) {
    if constexpr (PHASE == 2) {
      const int rows = rows_of(c);
      const float gt = SEL ? gate_readout<REV>(tab, t) : gp[t + 1];
      Frag<T> xf[KX / 32];
#pragma unroll
      for (int kq = 0; kq < KX / 32; ++kq)
        load_frag8(xf[kq], sX + t * LX + 32 * kq + 8 * g);
      f32x4 pt[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (sb <= tb) {
#pragma unroll
          for (int kq = 0; kq < KX / 32; ++kq) {
            Frag<T> fa;
            load_frag8(fa, sY + (16 * sb + li) * LX + 32 * kq + 8 * g);
            acc = mma(fa, xf[kq], acc);
          }
        }
        if constexpr (SEL) {
          gate_scores<REV>(acc, tab, t, sb, g);
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int s_ = 16 * sb + 4 * g + rr;
            acc[rr] = s_ <= t ? acc[rr] * (DECAY ? bdec * gp[s_ <= t ? t - s_ : 0]
                                                 : 1.f)
                              : 0.f;
          }
        }
        pt[sb] = acc;
      }
      Frag<T> pf[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        frag_from_acc(pf[kp], pt[2 * kp], pt[2 * kp + 1]);
      const int64_t row = row0_of(c) + (REV && t < rows ? rows - 1 - t : t);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jb = 4 * jh + jj;
        f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          if (2 * kp <= tb) {
            Frag<T> zf;
            load_frag_tr44(zf, sZ, LZ, 32 * kp, 16 * jb, g, li);
            an = mma(zf, pf[kp], an);
          }
        }
#pragma unroll
        for (int kq = 0; kq < KX / 32; ++kq) {
          Frag<T> fa;
          load_frag8(fa, sST + (16 * jb + li) * LX + 32 * kq + 8 * g);
          ai = mma(fa, xf[kq], ai);
        }
        const f32x4 o = an + gt * ai;
        if (t < rows) {
          // dq (elu + 1): phi'(q) from the raw q row staged with the chunk
          const u32x2 qr =
              PFI ? *reinterpret_cast<const u32x2 *>(sP + t * LZ + 16 * jb + 4 * g)
                  : u32x2{0u, 0u};
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float xin =
                PFI ? (r % 2 == 0 ? bf16_lo(qr[r / 2]) : bf16_hi(qr[r / 2]))
                    : 0.f;
            x[r] = PFI ? o[r] * dphi(xin, true) : o[r];
          }
          store4(res + row * D + 16 * jb + 4 * g, x[0], x[1], x[2], x[3]);
        }
      }
    }
    state_update(c);
    __syncthreads();  // the tile set is free again
    stage(c + 1);
    load(c + 2);
    if constexpr (PHASE == 2) publish();
    __syncthreads();
  }
  if constexpr (PHASE == 1) {
    float *dst = slot(seg);
#pragma unroll
    for (int fb = 0; fb < NT; ++fb)
      *reinterpret_cast<f32x4 *>(dst + fb * 256) = S[fb];
    if (SEL && tid == 0) *seg_total(a, units, ROLE, unit, seg) = segl;
  }
}

// The dk and dv readouts fused (PHASE 2).  Both roles run backwards through
// the sequence over the same weights and share every operand: dk takes
// queries V+, keys G~, values Q'; dv queries K', keys Q', values G.  Their
// states are transposes of each other: S_dv = (the first d rows of
// S_dk)^T, both sums of w G~^T Q' over the rows already passed.  So one
// workgroup stages V+, G~, Q', K' and the raw k rows (whose phi'(k) scales
// dk) once per chunk, keeps S_dk (the dk role's state and aggregates, whose
// PHASE 1 is unchanged) and reads both outputs out of one S_dk^T copy: dk's
// inter-chunk term takes its rows, dv's its columns through transposing
// reads.  Wave w = 4 jh + tb reads out strip tb of both outputs for column
// blocks 4 jh .. 4 jh + 3.
constexpr size_t kDkvLds =
    sizeof(bf16) * (2 * SShape<bf16, kRoleDK>::SX + 3 * SShape<bf16, kRoleDK>::SZ +
                    SShape<bf16, kRoleDK>::SST) +
    sizeof(float) * SShape<bf16, kRoleDK>::TAB;

template <bool DECAY, bool ELU, bool SEL = false>
__device__ __forceinline__ void seg_dkv(const BwdArgs &a, int64_t units,
                                        int64_t unit, int seg,
                                        unsigned char *smem) {
  using T = bf16;
  using F = SShape<T, kRoleDK>;
  const int nseg = a.nseg;
  constexpr int D = F::D, C = kBC, KX = F::KX, LX = F::LX, LZ = F::LZ;
  constexpr int NT = F::NT, KG = backward_gwidth(D);
  T *sV = reinterpret_cast<T *>(smem);  // V+ rows: dk's queries
  T *sG = sV + F::SX;                   // G~ rows: dk's keys, dv's values
  T *sQ = sG + F::SX;                   // Q': dk's values, dv's keys
  T *sK = sQ + F::SZ;                   // K': dv's queries
  T *sKr = sK + F::SZ;                  // raw k: phi'(k) of dk's outputs
  T *sST = sKr + F::SZ;                 // S_dk^T: row f of Q', column c of G~
  float *gp = reinterpret_cast<float *>(sST + F::SST);  // g^0 .. g^C
  float *tab = gp;  // SEL: the chunk's table (gate_table) instead

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tb = w % 4, jh = w / 4;
  const int h = static_cast<int>(unit % a.H);
  constexpr bool HD = DECAY && !SEL;  // one decay per head
  const float gdec = HD ? a.decay[h] : 1.f, bdec = HD ? 1.f - gdec : 1.f;
  const float lg = log2f(gdec);
  if constexpr (!SEL)
    for (int i = tid; i <= C; i += kSThreads) gp[i] = pow_int(gdec, lg, i);
  const float *lb = SEL ? a.lam + unit * a.n : nullptr;
  float laml = 0.f;  // SEL, wave 0: lam of processing index `lane`

  const int64_t n = a.n;
  const T *qb = static_cast<const T *>(a.q) + unit * n * D;
  const T *kb = static_cast<const T *>(a.k) + unit * n * D;
  const T *vb = static_cast<const T *>(a.v) + unit * n * D;
  const T *gtb = static_cast<const T *>(a.gt) + unit * n * KG;
  T *dkb = static_cast<T *>(a.dk) + unit * n * D;
  T *dvb = static_cast<T *>(a.dv) + unit * n * D;

  // the zero padding columns of V+ (G~ rows are copied whole, V+'s ones
  // columns are written per chunk)
  for (int i = tid; i < C * (KX - D - 2); i += kSThreads) {
    const int row = i / (KX - D - 2), col = D + 2 + i % (KX - D - 2);
    sV[row * LX + col] = from_f32<T>(0.f);
  }

  // processing steps: step c is physical chunk nch - 1 - c, its rows reversed
  const int nch = static_cast<int>((n + C - 1) / C);
  const int cps = (nch + nseg - 1) / nseg;
  const int cb = seg * cps, ce = min(nch, cb + cps);
  auto rows_of = [&](int c) -> int {
    if (c >= ce) return 0;
    const int64_t r0 = static_cast<int64_t>(nch - 1 - c) * C;
    return static_cast<int>(min<int64_t>(C, n - r0));
  };
  auto row0_of = [&](int c) -> int64_t {
    return c >= ce ? 0 : static_cast<int64_t>(nch - 1 - c) * C;
  };

  // register ring, one chunk ahead: G~, v, and the raw q and k rows
  using SG = BSlab<T, KG, KG, kSThreads>;
  using SD = BSlab<T, D, D, kSThreads>;
  SG rg;
  SD rv, rq, rk;
  auto load = [&](int c) {
    const int64_t r0 = row0_of(c);
    const int rows = rows_of(c);
    rg.load(gtb, r0, rows, 0, tid);
    rv.load(vb, r0, rows, 0, tid);
    rq.load(qb, r0, rows, 0, tid);
    rk.load(kb, r0, rows, 0, tid);
    if constexpr (SEL) {
      if (w == 0) {  // rows past the end are out of the resource: lam 0
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(lb + r0, static_cast<unsigned>(rows) * sizeof(float));
        const int rr = lane < rows ? rows - 1 - lane : lane;
        laml = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       r, static_cast<unsigned>(rr) * 4u, 0, 0));
      }
    }
  };
  auto put_phi = [&](const SD &sl, T *dst, auto trow, int rows) {
#pragma unroll
    for (int i = 0; i < SD::PER; ++i) {
      const int p = tid + SD::THREADS * i;
      if (SD::EXACT || p < SD::PIECES) {
        const int r = p / SD::PPR;
        u32x4 y = sl.v[i];
        if constexpr (ELU) {
          float f[SD::VEC];
          piece_to_f32<T>(sl.v[i], f);
#pragma unroll
          for (int e = 0; e < SD::VEC; ++e)
            f[e] = r < rows ? elu_plus_one_fast(f[e]) : 0.f;
          y = f32_to_piece<T>(f);
        }
        *reinterpret_cast<u32x4 *>(dst + trow(r) * LZ + (p % SD::PPR) * SD::VEC) =
            y;
      }
    }
  };
  auto put_raw = [&](const SD &sl, T *dst, auto trow) {
#pragma unroll
    for (int i = 0; i < SD::PER; ++i) {
      const int p = tid + SD::THREADS * i;
      if (SD::EXACT || p < SD::PIECES)
        *reinterpret_cast<u32x4 *>(dst + trow(p / SD::PPR) * LZ +
                                   (p % SD::PPR) * SD::VEC) = sl.v[i];
    }
  };
  auto put = [&](const auto &sl, T *dst, auto trow) {
    using S = std::remove_cv_t<std::remove_reference_t<decltype(sl)>>;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
      const int p = tid + S::THREADS * i;
      if (S::EXACT || p < S::PIECES)
        *reinterpret_cast<u32x4 *>(dst + trow(p / S::PPR) * LX +
                                   (p % S::PPR) * S::VEC) = sl.v[i];
    }
  };
  auto stage = [&](int c) {
    const int rows = rows_of(c);
    auto trow = [&](int r) { return r < rows ? rows - 1 - r : r; };
    if constexpr (SEL)
      if (w == 0) gate_table<true>(laml, tab, lane, rows);
    put(rg, sG, trow);
    put(rv, sV, trow);
    if (tid < C) {
      const int t = trow(tid);
      const T one = from_f32<T>(tid < rows ? 1.f : 0.f);
      sV[t * LX + D] = one;
      sV[t * LX + D + 1] = one;
    }
    put_phi(rq, sQ, trow, rows);
    put_phi(rk, sK, trow, rows);
    if constexpr (ELU) put_raw(rk, sKr, trow);
  };

  // this wave's part of S_dk: column block w of Q', all NT tiles of G~;
  // the entering state sums the dk role's aggregates before this segment
  f32x4 S[NT];
#pragma unroll
  for (int fb = 0; fb < NT; ++fb) S[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // (SEL: carried over the segments between by their sums of log2 gamma)
  float between = 0.f;
  for (int i = 0; i < seg; ++i) {
    const int sg = SEL ? seg - 1 - i : i;
    const float wgt =
        SEL  ? __builtin_amdgcn_exp2f(between)
        : HD ? pow_int(gdec, lg, static_cast<int64_t>(seg - sg - 1) * cps * C)
             : 1.f;
    if constexpr (SEL) between += *seg_total(a, units, kRoleDK, unit, sg);
    const float *src = a.agg +
                       ((static_cast<int64_t>(kRoleDK) * units + unit) * nseg +
                        sg) * kSegSlot +
                       (w * kSegTiles) * 256 + lane * 4;
#pragma unroll
    for (int fb = 0; fb < NT; ++fb)
      S[fb] += wgt * *reinterpret_cast<const f32x4 *>(src + fb * 256);
  }
  auto publish = [&]() {  // S_dk^T rows 16 w .. + 15
#pragma unroll
    for (int fb = 0; fb < NT; ++fb)
      store4(sST + (16 * w + li) * LX + 16 * fb + 4 * g, S[fb][0], S[fb][1],
             S[fb][2], S[fb][3]);
  };
  auto state_update = [&](int c) {  // S_dk <- g^r S_dk + sum w G~^T Q'
    const int rows = rows_of(c);
    const float gr = SEL ? tab[3 * C] : gp[rows];
    f32x4 wlo[C / 32], whi[C / 32];
    if constexpr (SEL) {
      gate_update(tab, g, wlo, whi);
    } else if constexpr (DECAY) {
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s0 = 32 * kb2 + 8 * g + e, s1 = s0 + 4;
          wlo[kb2][e] = s0 < rows ? bdec * gp[rows - 1 - s0] : 0.f;
          whi[kb2][e] = s1 < rows ? bdec * gp[rows - 1 - s1] : 0.f;
        }
    }
    Frag<T> bf[C / 32];
#pragma unroll
    for (int kb2 = 0; kb2 < C / 32; ++kb2) {
      load_frag_tr8(bf[kb2], sQ, LZ, 32 * kb2, 16 * w, g, li);
      if constexpr (DECAY) frag_scale(bf[kb2], wlo[kb2], whi[kb2]);
    }
#pragma unroll
    for (int fb = 0; fb < NT; ++fb) {
      f32x4 acc = S[fb] * gr;
#pragma unroll
      for (int kb2 = 0; kb2 < C / 32; ++kb2) {
        Frag<T> af;
        load_frag_tr8(af, sG, LX, 32 * kb2, 16 * fb, g, li);
        acc = mma(af, bf[kb2], acc);
      }
      S[fb] = acc;
    }
  };

  const int t = 16 * tb + li;  // the query row this lane reads out
  // masked, decay-weighted scores P^T (keys s = 16 sb + 4 g + r of the
  // chunk, this lane's query t) from the key rows of sY against xf
  auto scores = [&](Frag<T>(&pf)[2], const T *sY, int ly, const Frag<T> *xf,
                    auto nk) {
    constexpr int NK = decltype(nk)::value;
    f32x4 pt[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (sb <= tb) {
#pragma unroll
        for (int kq = 0; kq < NK; ++kq) {
          Frag<T> fa;
          load_frag8(fa, sY + (16 * sb + li) * ly + 32 * kq + 8 * g);
          acc = mma(fa, xf[kq], acc);
        }
      }
      if constexpr (SEL) {
        gate_scores<true>(acc, tab, t, sb, g);
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int s_ = 16 * sb + 4 * g + rr;
          acc[rr] = s_ <= t ? acc[rr] * (DECAY ? bdec * gp[s_ <= t ? t - s_ : 0]
                                               : 1.f)
                            : 0.f;
        }
      }
      pt[sb] = acc;
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
      frag_from_acc(pf[kp], pt[2 * kp], pt[2 * kp + 1]);
  };

  load(cb);
  __syncthreads();  // gp and the padding columns ready
  stage(cb);
  load(cb + 1);
  publish();
  __syncthreads();

  for (int c = cb; c < ce; ++c) {
    const int rows = rows_of(c);
    const float gt = SEL ? gate_readout<true>(tab, t) : gp[t + 1];
    const int64_t row = row0_of(c) + (t < rows ? rows - 1 - t : t);
    // ---- dk: queries V+ (KX wide), keys G~, values Q'
    {
      Frag<T> xf[KX / 32];
#pragma unroll
      for (int kq = 0; kq < KX / 32; ++kq)
        load_frag8(xf[kq], sV + t * LX + 32 * kq + 8 * g);
      Frag<T> pf[2];
      scores(pf, sG, LX, xf, std::integral_constant<int, KX / 32>{});
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jb = 4 * jh + jj;
        f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          if (2 * kp <= tb) {
            Frag<T> zf;
            load_frag_tr44(zf, sQ, LZ, 32 * kp, 16 * jb, g, li);
            an = mma(zf, pf[kp], an);
          }
        }
#pragma unroll
        for (int kq = 0; kq < KX / 32; ++kq) {
          Frag<T> fa;
          load_frag8(fa, sST + (16 * jb + li) * LX + 32 * kq + 8 * g);
          ai = mma(fa, xf[kq], ai);
        }
        const f32x4 o = an + gt * ai;
        if (t < rows) {
          // phi'(k) from the raw k row staged with the chunk
          const u32x2 kr =
              ELU ? *reinterpret_cast<const u32x2 *>(sKr + t * LZ + 16 * jb + 4 * g)
                  : u32x2{0u, 0u};
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float xin =
                ELU ? (r % 2 == 0 ? bf16_lo(kr[r / 2]) : bf16_hi(kr[r / 2]))
                    : 0.f;
            x[r] = ELU ? o[r] * dphi(xin, true) : o[r];
          }
          store4(dkb + row * D + 16 * jb + 4 * g, x[0], x[1], x[2], x[3]);
        }
      }
    }
    // ---- dv: queries K', keys Q', values G (the first d columns of G~);
    // the state term reads S_dv = S_dk^T through transposing reads of sST
    {
      Frag<T> xf[D / 32];
#pragma unroll
      for (int kq = 0; kq < D / 32; ++kq)
        load_frag8(xf[kq], sK + t * LZ + 32 * kq + 8 * g);
      Frag<T> pf[2];
      scores(pf, sQ, LZ, xf, std::integral_constant<int, D / 32>{});
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jb = 4 * jh + jj;
        f32x4 an = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          if (2 * kp <= tb) {
            Frag<T> zf;
            load_frag_tr44(zf, sG, LX, 32 * kp, 16 * jb, g, li);
            an = mma(zf, pf[kp], an);
          }
        }
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) {
          Frag<T> fa;
          load_frag_tr8(fa, sST, LX, 32 * kq, 16 * jb, g, li);
          ai = mma(fa, xf[kq], ai);
        }
        const f32x4 o = an + gt * ai;
        if (t < rows)
          store4(dvb + row * D + 16 * jb + 4 * g, o[0], o[1], o[2], o[3]);
      }
    }
    state_update(c);
    __syncthreads();  // the tile set is free again
    stage(c + 1);
    load(c + 2);
    publish();
    __syncthreads();
  }
}

// The aggregates launch (PHASE 1) runs two workgroups per CU (four waves
// per SIMD: at most 128 VGPRs); the readout one.
template <bool DECAY, bool ELU, int PHASE, bool SEL = false>
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(
    PHASE == 1 ? 4 : 1))) void la_bwd_seg_kernel(BwdArgs a, int64_t units) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nseg = a.nseg;
  const int64_t per_role = units * nseg;
  const int role = static_cast<int>(blockIdx.x / per_role);
  const int64_t rem = blockIdx.x % per_role;
  const int64_t unit = rem / nseg;
  const int seg = static_cast<int>(rem % nseg);
  // the last segment's aggregate is never read
  if (PHASE == 1 && seg == nseg - 1) return;
  // role 0: dq; role 1: the dk aggregates (PHASE 1), dk and dv (PHASE 2)
  if (role == kRoleDQ) {
    seg_role<bf16, kRoleDQ, DECAY, ELU, PHASE, SEL>(a, units, unit, seg, smem);
  } else {
    if constexpr (PHASE == 1)
      seg_role<bf16, kRoleDK, DECAY, ELU, 1, SEL>(a, units, unit, seg, smem);
    else
      seg_dkv<DECAY, ELU, SEL>(a, units, unit, seg, smem);
  }
}

template <bool DECAY, bool ELU, bool SEL = false>
hipError_t launch_seg(const BwdArgs &a, int64_t units, hipStream_t s) {
  const int nseg = a.nseg;
  constexpr size_t lds = std::max({SShape<bf16, kRoleDQ>::lds_bytes,
                                   SShape<bf16, kRoleDK>::lds_bytes,
                                   kDkvLds});
  constexpr size_t lds1 = std::max(SShape<bf16, kRoleDQ>::lds_bytes_agg,
                                   SShape<bf16, kRoleDK>::lds_bytes_agg);
  static_assert(lds <= 160 * 1024 && 2 * lds1 <= 160 * 1024,
                "LDS of one workgroup (two for the aggregates)");
  static const hipError_t once = [] {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&la_bwd_seg_kernel<DECAY, ELU, 1, SEL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds1));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(
        reinterpret_cast<const void *>(&la_bwd_seg_kernel<DECAY, ELU, 2, SEL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  }();
  if (once != hipSuccess) return once;
  const dim3 grid(static_cast<unsigned>(2 * units * nseg)), block(kSThreads);
  if (nseg > 1) {
    hipLaunchKernelGGL((la_bwd_seg_kernel<DECAY, ELU, 1, SEL>), grid, block, lds1,
                       s, a, units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((la_bwd_seg_kernel<DECAY, ELU, 2, SEL>), grid, block, lds, s, a,
                     units);
  return hipGetLastError();
}

// All roles in one launch: blocks [0, units nq) take dq, the next units nq
// dk, the last units nv dv (nq = d'/16, nv = d/16).  Within a role the
// blocks of one unit get indices of one XCD (workgroups are dispatched to
// the 8 XCDs round-robin), so the rows they all read come from its L2.
// PART 0 runs all roles; the Performer map (d' > d) runs the dq and dk
// roles (PART 1) and the dv role (PART 2) as two launches, since dv's
// d'-wide tiles need more than twice the LDS of the others, which then fit
// four workgroups to a compute unit.
template <typename T, int DF, int PART>
constexpr int bwd_waves() {
  return sizeof(T) != 2 ? 1 : PART == 1 && DF > 128 ? 4 : DF <= 128 ? 3 : 2;
}
template <typename T, int D, int DF, bool DECAY, bool ELU, bool FG = false,
          bool SEL = false, int PART = 0>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(
    bwd_waves<T, DF, PART>())))
void la_bwd_kernel(BwdArgs a, int64_t units) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int nq = DF / 16, nv = D / 16;
  const int64_t cq = units * nq;
  const int64_t b = PART == 2 ? blockIdx.x + 2 * cq : blockIdx.x;
  const int role = b < cq ? kRoleDQ : b < 2 * cq ? kRoleDK : kRoleDV;
  int64_t i = role == kRoleDQ ? b : role == kRoleDK ? b - cq : b - 2 * cq;
  const int nblk = role == kRoleDV ? nv : nq;
  const int64_t span = units * nblk;
  if (span % 8 == 0) i = (i % 8) * (span / 8) + i / 8;
  const int64_t unit = i / nblk;
  const int blk = static_cast<int>(i % nblk);
  if constexpr (PART == 2) {
    bwd_role<T, D, DF, kRoleDV, DECAY, ELU, FG, SEL>(a, unit, blk, smem);
  } else {
    if (role == kRoleDQ)
      bwd_role<T, D, DF, kRoleDQ, DECAY, ELU, FG, SEL>(a, unit, blk, smem);
    else if (role == kRoleDK)
      bwd_role<T, D, DF, kRoleDK, DECAY, ELU, FG, SEL>(a, unit, blk, smem);
    else if constexpr (PART == 0)
      bwd_role<T, D, DF, kRoleDV, DECAY, ELU, FG, SEL>(a, unit, blk, smem);
  }
}

template <typename T, int D, bool ELU>
hipError_t launch_prep(const BwdArgs &a, int64_t units, hipStream_t s) {
  constexpr int RPB = kBThreads / (D / (16 / static_cast<int>(sizeof(T))));
  const int64_t steps = (units * a.n + RPB - 1) / RPB;
  const unsigned grid =
      static_cast<unsigned>(std::min<int64_t>(steps, int64_t{kCUs} * 16));
  hipLaunchKernelGGL((la_bwd_prep_kernel<T, D, ELU>), dim3(grid),
                     dim3(kBThreads), 0, s, a, units * a.n);
  return hipGetLastError();
}

template <typename T, int D, int DF, bool DECAY, bool ELU, bool FG = false,
          bool SEL = false>
hipError_t launch_all(const BwdArgs &a, int64_t units, hipStream_t s) {
  if constexpr (std::is_same_v<T, bf16> && D == kSegD && DF == D) {
    if (a.nseg > 0) {
      // segmented roles map k, q themselves: the preparation pass writes
      // only G~
      hipError_t e = launch_prep<T, D, false>(a, units, s);
      if (e != hipSuccess) return e;
      return launch_seg<DECAY, ELU, SEL>(a, units, s);
    }
  }
  hipError_t e = launch_prep<T, D, ELU>(a, units, s);
  if (e != hipSuccess) return e;
  using FQ = BShape<T, D, DF, kRoleDQ, DECAY, SEL>;
  using FK = BShape<T, D, DF, kRoleDK, DECAY, SEL>;
  using FV = BShape<T, D, DF, kRoleDV, DECAY, SEL>;
  // one launch of PART with lds bytes and blocks workgroups
  auto run = [&](auto part, size_t lds, int64_t blocks) -> hipError_t {
    constexpr int P = decltype(part)::value;
    auto *k = &la_bwd_kernel<T, D, DF, DECAY, ELU, FG, SEL, P>;
    static const hipError_t once = hipFuncSetAttribute(
        reinterpret_cast<const void *>(k),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (once != hipSuccess) return once;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBThreads), lds, s, a, units);
    return hipGetLastError();
  };
  if constexpr (FG) {
    constexpr size_t lds1 = std::max(FQ::lds_bytes, FK::lds_bytes);
    static_assert(lds1 <= 160 * 1024 && FV::lds_bytes <= 160 * 1024,
                  "LDS of one workgroup");
    e = run(std::integral_constant<int, 1>{}, lds1, units * 2 * (DF / 16));
    if (e != hipSuccess) return e;
    return run(std::integral_constant<int, 2>{}, FV::lds_bytes,
               units * (D / 16));
  } else {
    constexpr size_t lds =
        std::max({FQ::lds_bytes, FK::lds_bytes, FV::lds_bytes});
    static_assert(lds <= 160 * 1024, "LDS of one workgroup");
    return run(std::integral_constant<int, 0>{}, lds,
               units * (2 * (DF / 16) + D / 16));
  }
}

// Performer map ("Linear attention research 2026" page, Performer random
// features: phi_r(x) = exp(x . omega_r - |x|^2 / 2) / sqrt(m)), whose
// derivative is d phi_r / d x = phi_r(x) (omega_r - x): a feature gradient
// gx' becomes, per row,
//   gx = (gx' * phi(x)) omega^T - x sum_r gx'_r phi_r(x).
// For the queries the last sum is exactly zero: each output is unchanged
// when q'_t is scaled (q'_t mu_t / q'_t . nu_t), so q'_t . dq'_t = 0.  It is
// dropped there (with_sum = 0): computed from rounded operands it would
// only add the noise of a cancelling sum of d' terms.
// 64 rows per step: u = gx' * phi(x) ([row][r]) in LDS, the product
// u omega^T on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32: exact
// products, fp32 sums); each wave takes every fourth 16 x 16 output tile,
// whose columns are always the same one or two blocks of 16 rows of omega:
// their fragments are loaded once per workgroup and kept in registers (at
// most 64 values per lane for d * d' <= 16384), which leaves LDS to u and
// lets two workgroups share a compute unit.  Rows past the end are skipped.
constexpr int kPfRows = 64;
template <int D, int DF>
constexpr size_t pf_grad_lds() {
  return sizeof(float) * (static_cast<size_t>(kPfRows) * (DF + 4) + kPfRows);
}

template <typename T, int D, int DF>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(
    2))) void la_bwd_pf_grad_kernel(
    const T *__restrict__ xf, const float *__restrict__ gf,
    const T *__restrict__ x, T *__restrict__ dx,
    const float *__restrict__ omega, int64_t rows, int with_sum) {
  constexpr int PR = kPfRows, L = DF + 4;  // row stride of omega and u
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NT = (PR / 16) * (D / 16), TPW = NT / kBWaves;
  constexpr int TPR = DF / VEC;            // fill threads per row
  // column blocks of omega a wave's tiles use: tile w + kBWaves m has
  // column block (w + kBWaves m) % (D / 16), which is block j = that / 4
  // of the wave's own list w % (D / 16) + kBWaves j
  constexpr int NCB = D / 16, NB = (NCB + kBWaves - 1) / kBWaves;
  static_assert(DF % 32 == 0 && D % 16 == 0 && kBThreads % TPR == 0 &&
                    TPR <= kWave && NT % kBWaves == 0 &&
                    (NCB % kBWaves == 0 || kBWaves % NCB == 0),
                "tiling");
  extern __shared__ __align__(16) unsigned char smem[];
  float *u = reinterpret_cast<float *>(smem);   // [PR][L]
  float *su = u + PR * L;                       // [PR]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6, g = lane >> 4, li = lane & 15;
  Frag<float> of[NB][DF / 32];  // omega rows of the wave's column blocks
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int kb = 0; kb < DF / 32; ++kb)
      load_frag8(of[j][kb],
                 omega + (16 * (w % NCB + kBWaves * j) + li) * DF + 32 * kb +
                     8 * g);
  const int64_t nsteps = (rows + PR - 1) / PR;
  for (int64_t st = blockIdx.x; st < nsteps; st += gridDim.x) {
    const int64_t row0 = st * PR;
    __syncthreads();  // the previous step's u, su are read
    // fill: TPR consecutive threads take one row, VEC features each; the
    // loads of each batch of 4 rounds (of all, when there are fewer) are
    // issued before any is used
    constexpr int FA = PR * TPR / kBThreads;  // fill rounds
    constexpr int FH = FA > 4 ? FA / 4 : 1, FI = FA / FH;
    static_assert(PR * TPR % kBThreads == 0 && FA % FH == 0,
                  "whole fill rounds");
#pragma unroll
    for (int hf = 0; hf < FH; ++hf) {
    f32x4 gl[FI][VEC / 4];
    u32x4 xl[FI];
#pragma unroll
    for (int it = 0; it < FI; ++it) {
      const int p = tid + kBThreads * (FI * hf + it);
      const int rr = p / TPR, f0 = (p % TPR) * VEC;
      const int64_t off = (row0 + rr) * DF + f0;
      const bool in = row0 + rr < rows;
#pragma unroll
      for (int e = 0; e < VEC / 4; ++e)
        gl[it][e] = in ? *reinterpret_cast<const f32x4 *>(gf + off + 4 * e)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      xl[it] = in ? *reinterpret_cast<const u32x4 *>(xf + off)
                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < FI; ++it) {
      const int p = tid + kBThreads * (FI * hf + it);
      const int rr = p / TPR, f0 = (p % TPR) * VEC;
      float a[VEC], b[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) a[e] = gl[it][e / 4][e % 4];
      piece_to_f32<T>(xl[it], b);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const f32x4 ue = {a[e] * b[e], a[e + 1] * b[e + 1],
                          a[e + 2] * b[e + 2], a[e + 3] * b[e + 3]};
        *reinterpret_cast<f32x4 *>(u + rr * L + f0 + e) = ue;
        part += (ue[0] + ue[1]) + (ue[2] + ue[3]);
      }
      // the row's TPR threads are consecutive and aligned: sum them
      part = sum_group<TPR>(part);
      if (p % TPR == 0) su[rr] = with_sum ? part : 0.f;
    }
    }
    __syncthreads();
    f32x4 acc[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DF / 32; ++kb) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        // (w < kBWaves: block j of tile m is known at compile time)
        const int mt = (w + kBWaves * m) / NCB;
        const int j = NCB >= kBWaves ? m % (NCB / kBWaves) : 0;
        Frag<float> fa;
        load_frag8(fa, u + (16 * mt + li) * L + 32 * kb + 8 * g);
        acc[m] = mma(fa, of[j][kb], acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = w + kBWaves * m;
      const int mt = t / NCB, nt = t % NCB;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = 16 * mt + 4 * g + r;
        const int64_t row = row0 + rl;
        if (row < rows) {
          const int64_t o = row * D + 16 * nt + li;
          dx[o] = from_f32<T>(acc[m][r] - to_f32(x[o]) * su[rl]);
        }
      }
    }
  }
}

// Performer backward for one size: G~ (no features: K' and Q' are in the
// workspace already), the three roles by column blocks (dq', dk' to the
// workspace in fp32, dv to its output), then dq and dk through the map.
template <typename T, int D, int DF>
hipError_t launch_pf(const BwdArgs &a, int64_t units, hipStream_t s) {
  // (launch_all runs the preparation pass first)
  hipError_t e =
      a.lam     ? launch_all<T, D, DF, true, false, true, true>(a, units, s)
      : a.decay ? launch_all<T, D, DF, true, false, true>(a, units, s)
                : launch_all<T, D, DF, false, false, true>(a, units, s);
  if (e != hipSuccess) return e;
  constexpr size_t lds = pf_grad_lds<D, DF>();
  static_assert(lds <= 160 * 1024, "LDS of the conversion pass");
  static const hipError_t once = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&la_bwd_pf_grad_kernel<T, D, DF>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (once != hipSuccess) return once;
  const int64_t rows = units * a.n;
  const unsigned grid = static_cast<unsigned>(
      std::min<int64_t>((rows + kPfRows - 1) / kPfRows, int64_t{kCUs} * 4));
  hipLaunchKernelGGL((la_bwd_pf_grad_kernel<T, D, DF>), dim3(grid),
                     dim3(kBThreads), lds, s, static_cast<const T *>(a.qf),
                     static_cast<const float *>(a.dqf), static_cast<const T *>(a.q),
                     static_cast<T *>(a.dq), a.omega, rows, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((la_bwd_pf_grad_kernel<T, D, DF>), dim3(grid),
                     dim3(kBThreads), lds, s, static_cast<const T *>(a.kf),
                     static_cast<const float *>(a.dkf), static_cast<const T *>(a.k),
                     static_cast<T *>(a.dk), a.omega, rows, 1);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_pf_d(const BwdArgs &a, int64_t units, int df, hipStream_t s) {
  switch (df) {
    case 32: return launch_pf<T, D, 32>(a, units, s);
    case 64: return launch_pf<T, D, 64>(a, units, s);
    case 128: return launch_pf<T, D, 128>(a, units, s);
    case 256:
      if constexpr (D * 256 <= 16384) return launch_pf<T, D, 256>(a, units, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_pf_t(const BwdArgs &a, int64_t units, int d, int df,
                       hipStream_t s) {
  switch (d) {
    case 32: return launch_pf_d<T, 32>(a, units, df, s);
    case 64: return launch_pf_d<T, 64>(a, units, df, s);
    case 128: return launch_pf_d<T, 128>(a, units, df, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_d(const BwdArgs &a, int64_t units, hipStream_t s) {
  if (a.lam)
    return a.elu1 ? launch_all<T, D, D, true, true, false, true>(a, units, s)
                  : launch_all<T, D, D, true, false, false, true>(a, units, s);
  if (a.decay)
    return a.elu1 ? launch_all<T, D, D, true, true>(a, units, s)
                  : launch_all<T, D, D, true, false>(a, units, s);
  return a.elu1 ? launch_all<T, D, D, false, true>(a, units, s)
                : launch_all<T, D, D, false, false>(a, units, s);
}

template <typename T>
hipError_t launch_t(const BwdArgs &a, int64_t units, int d, hipStream_t s) {
  switch (d) {
    case 16: return launch_d<T, 16>(a, units, s);
    case 32: return launch_d<T, 32>(a, units, s);
    case 64: return launch_d<T, 64>(a, units, s);
    case 128: return launch_d<T, 128>(a, units, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool backward_supported(int d, int d_feat) {
  return d == d_feat && (d == 16 || d == 32 || d == 64 || d == 128);
}

bool backward_performer_supported(int d, int d_feat) {
  return (d == 32 || d == 64 || d == 128) &&
         (d_feat == 32 || d_feat == 64 || d_feat == 128 || d_feat == 256) &&
         d * d_feat <= 16384;
}

hipError_t launch_backward_performer(const BwdArgs &a, int64_t units, int d,
                                     int d_feat, int dtype, hipStream_t s) {
  if (!backward_performer_supported(d, d_feat)) return hipErrorInvalidValue;
  return dtype == 1 ? launch_pf_t<bf16>(a, units, d, d_feat, s)
                    : launch_pf_t<float>(a, units, d, d_feat, s);
}

int backward_segments(int64_t units, int64_t n, int d, int dtype) {
  if (dtype != 1 || d != kSegD || units <= 0 || n <= 0) return 0;
  // two roles (dq; dk with dv) x units x segments workgroups of one per
  // CU: about two rounds of the CUs, at most 16 segments, whole chunks each
  const int64_t nch = (n + kBC - 1) / kBC;
  int64_t k = (kCUs + units - 1) / units;
  if (k > 16) k = 16;
  if (k > nch) k = nch;
  if (k < 1) k = 1;
  // segments of whole chunks: the last non-empty one decides the count
  const int64_t cps = (nch + k - 1) / k;
  return static_cast<int>((nch + cps - 1) / cps);
}

size_t backward_agg_floats(int64_t units, int nseg) {
  // aggregates of the dq and dk roles (the fused dk and dv readout takes
  // dk's)
  // and, after them, each segment's sum of log2 gamma (a decay per
  // position; unused otherwise)
  return nseg > 1 ? static_cast<size_t>(2 * units * nseg) * (kSegSlot + 1)
                  : 0;
}

hipError_t launch_backward(const BwdArgs &a, int64_t units, int d, int dtype,
                           hipStream_t s) {
  return dtype == 1 ? launch_t<bf16>(a, units, d, s)
                    : launch_t<float>(a, units, d, s);
}

}  // namespace la
