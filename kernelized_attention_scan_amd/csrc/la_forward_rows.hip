// Forward with a decay per state row: the carry scan over segment
// aggregates, the segment plan and the instance lookup.
#include "la_forward_rows.h"
#include "la_internal.h"

namespace la {

// Each segment's incoming state from the aggregates, in place: slot j of a
// unit becomes the state before segment j, for j < nseg; slot nseg receives
// the sum through segment nsum - 1 (the total, for the non-causal form, which
// also writes it to mu_out / nu_out in their natural layouts when given).
// One thread per state element (accumulator order: ((jb nft + i) 64 + lane)
// 4 + r holds row 16 i + 4 (lane / 16) + r, column 16 jb + lane % 16) or nu
// entry, sequential over the segments:
//   in_0 = 0,  in_{j+1} = 2^(D_j[f]) in_j + A_j
// with D_j the segment's summed log2 decay of row f.
__global__ __launch_bounds__(256) void la_fwd_rows_carry_kernel(
    float *agg, int nseg, int nsum, int slot, int nstate, int dfp, int nft,
    int d, int df, float *mu_out, float *nu_out) {
  const int nb = (nstate + dfp + 255) / 256;  // blocks per unit
  const int64_t unit = blockIdx.x / nb;
  const int x = static_cast<int>(blockIdx.x % nb) * 256 + threadIdx.x;
  if (x >= nstate + dfp) return;
  int f, e = -1;
  if (x < nstate) {
    const int r = x & 3, ln = (x >> 2) & 63, rest = x >> 8;
    f = 16 * (rest % nft) + 4 * (ln >> 4) + r;
    e = 16 * (rest / nft) + (ln & 15);
  } else {
    f = x - nstate;
  }
  float *base = agg + unit * (nseg + 1) * static_cast<int64_t>(slot);
  float s = 0.f;
  for (int j = 0; j < nseg; ++j) {
    float *p = base + j * static_cast<int64_t>(slot);
    const float av = p[x];
    const float dl = p[nstate + dfp + f];
    p[x] = s;
    if (j < nsum) s = s * exp2f(dl) + av;
  }
  base[nseg * static_cast<int64_t>(slot) + x] = s;
  if (mu_out && f < df) {
    if (e >= 0)
      mu_out[(unit * df + f) * d + e] = s;
    else
      nu_out[unit * df + f] = s;
  }
}

// About two workgroups per compute unit in all, whole chunks per segment,
// at most kMaxSegments segments per unit.
int row_segments(int64_t units, int64_t n) {
  const int64_t nch = (n + kRowChunk - 1) / kRowChunk;
  if (units <= 0 || nch <= 0) return 1;
  int64_t k = (2 * kCUs + units - 1) / units;
  if (k > kMaxSegments) k = kMaxSegments;
  if (k > nch) k = nch;
  if (k < 1) k = 1;
  const int64_t cps = (nch + k - 1) / k;
  return static_cast<int>((nch + cps - 1) / cps);
}

const RowOps *row_ops(int d, int d_feat, int dtype) {
  return dtype == 1 ? row_ops_bf16(d, d_feat) : row_ops_f32(d, d_feat);
}

}  // namespace la
