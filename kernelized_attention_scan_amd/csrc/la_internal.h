// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

// At most this many sequence segments per (batch, head) unit.
constexpr int kMaxSegments = 16;

// Compute units of an MI355X.  A forward is split into about
// kCUs * (workgroups per CU of its instance) workgroups; a sequence is split
// into several segments only when there are fewer (batch, head) units than
// that, never more than kMaxTargetGroups.
constexpr int kCUs = 256;
constexpr int kMaxTargetGroups = 512;

// Synchronisation area at the start of the workspace of a multi-segment
// forward (32-bit words, zero between calls).  Its size is fixed, so that
// whatever sizes the calls sharing a workspace have, no call's scratch ever
// lands on another call's flags:
//   words [0, kSyncHeaderWords): header; word kSyncStatusWord collects
//     kSyncStatusTimeout (a wait for another segment's aggregate gave up;
//     the outputs of that segment are NaN) and kSyncStatusCorrupt (a
//     segment ticket was out of range: the area was not zero at the start);
//     kernels only ever set bits there, la_workspace_check reads and clears
//     it;
//   then one line of kSyncLineWords per (batch, head) unit, for up to
//     kMaxTargetGroups units: word s is the "aggregate of segment s published"
//     flag, word kSyncTicketWord hands out causal segment indices in start
//     order, word kSyncDoneWord counts the segments done waiting (the last
//     one clears the line), and the two words from kSyncXccWord record, 4
//     bits per segment, the XCD (1 + its id) each segment runs on.
constexpr int kSyncHeaderWords = 64;
constexpr int kSyncStatusWord = 8;
constexpr unsigned kSyncStatusTimeout = 1u;
constexpr unsigned kSyncStatusCorrupt = 2u;
// Polls of an exchange wait before it gives up, by default (about a second
// or more; la_set_exchange_spin_limit changes it for diagnostics).
constexpr unsigned kDefaultSpinLimit = 1u << 22;
constexpr int kSyncLineWords = 32;
constexpr int kSyncDoneWord = kMaxSegments;
constexpr int kSyncTicketWord = kMaxSegments + 1;
constexpr int kSyncXccWord = kMaxSegments + 2;
constexpr size_t kSyncBytes =
    sizeof(unsigned) * (kSyncHeaderWords + kMaxTargetGroups * kSyncLineWords);
static_assert(kSyncXccWord + 1 < kSyncLineWords, "sync line too short");
static_assert(kMaxSegments <= 16, "4-bit XCD records: two words per line");
static_assert(kSyncBytes % 256 == 0, "sync area keeps the states aligned");

// Arguments of the chunked forward kernels.
struct FwdArgs {
  const void *q, *k, *v;
  void *out;
  const float *decay;   // [H] or null
  float *states;        // [units][nseg][slot] segment aggregates, or null
  unsigned *sync;       // synchronisation area (zero between launches)
  int H;
  int64_t n;
  int64_t seg_len;      // multiple of the chunk length
  int nseg;
  int elu1;             // 1: phi = elu + 1 on q, k; 0: q, k are features
  const float *omega;   // [d][d_feat] for the fused Performer map, else null
  float *mu_out;        // [units][d_feat][d] final state, or null
  float *nu_out;        // [units][d_feat] final normaliser (with mu_out)
  unsigned spin_limit;  // polls of an exchange wait before it gives up
  // per-position decay: log gamma [units][n], or null; and (several
  // segments) each segment's sum of log2 gamma [units][nseg] in the
  // workspace
  const float *log_decay;
  float *seg_log;
  // training forward: q'_j . nu_j of every row [units][n] (causal), or null
  float *den_out;
};

// Launch set of one (storage type, d, d_feat) instance of the chunked forward.
struct FwdOps {
  int C;              // chunk rows
  int slot_floats;    // floats per fp32 state slot
  bool decay_ok;      // the decayed variant fits in LDS too
  bool sel_ok;        // the per-position decay variant fits in LDS too
  int vsplit;         // computations per unit (value column parts), 1 or 2
  // Enqueue the fused forward.
  hipError_t (*run)(const FwdArgs &args, int64_t units, int causal,
                    hipStream_t stream);
};

// nullptr when the combination is not built (unsupported size or LDS).
const FwdOps *fwd_ops_bf16(int d, int d_feat);
const FwdOps *fwd_ops_f32(int d, int d_feat);
// The forward with the Performer map fused into it (q, k of width d are
// mapped to d_feat random features on chip); bf16 storage only.  nullptr
// when not built for these sizes.
const FwdOps *fwd_ops_bf16_performer(int d, int d_feat);

// Arguments of the chunked forward with a decay per state row (one value
// per row and head, or one per position and row).
struct RowArgs {
  const void *q, *k, *v;  // [units][n][d_feat], [units][n][d_feat], [units][n][d]
  void *out;              // [units][n][d]
  const float *lam;       // log g: [H][d_feat] or [units][n][d_feat]
  int per_position;       // 0: lam is [H][d_feat]; 1: [units][n][d_feat]
  int H;
  int64_t n;
  int64_t seg_len;        // multiple of kRowChunk
  int nseg;
  int elu1;               // phi = elu + 1 on q, k (else they are features)
  int skip_last;          // set by the launcher for the aggregate launch
  float *agg;             // [units][nseg + 1][slot_floats] aggregates
  float *mu_out, *nu_out; // final state (both or neither), or null
};
constexpr int kRowChunk = 16;

// Launch set of one (storage type, d, d_feat) instance of that forward.
struct RowOps {
  int slot_floats;  // floats per aggregate slot
  // Enqueue the aggregate, carry and readout launches (the first two only
  // for several segments or the non-causal form).
  hipError_t (*run)(const RowArgs &args, int64_t units, int causal,
                    hipStream_t stream);
};
// nullptr for sizes that are not built; dtype 0 fp32, 1 bf16.
const RowOps *row_ops(int d, int d_feat, int dtype);
const RowOps *row_ops_bf16(int d, int d_feat);
const RowOps *row_ops_f32(int d, int d_feat);
// Segments per unit of that forward.
int row_segments(int64_t units, int64_t n);

// Feature map launchers.  dtype codes: 0 fp32, 1 bf16.
hipError_t launch_featmap_elementwise(const void *x, void *y, int64_t count,
                                      int elu1, int in_dt, int out_dt,
                                      hipStream_t stream);
// Returns hipErrorInvalidValue for sizes it was not built for.
hipError_t launch_featmap_performer(const void *x, void *y, const float *omega,
                                    int64_t rows, int d, int m, int in_dt,
                                    int out_dt, hipStream_t stream);

// Zero count floats (a fill kernel, so it can be captured in a graph).
hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t stream);

// Decode step launcher (map: 0 identity, 1 elu1, 2 performer).  With
// ld_layout < 0, decay is [H] or null; else it holds log gamma in that
// la_decay_layout (the gated form).
hipError_t launch_decode(float *mu, float *nu, const void *q, const void *k,
                         const void *v, void *out, int64_t units, int H, int d,
                         int d_feat, int map, const float *omega,
                         const float *decay, int dtype, hipStream_t stream,
                         int ld_layout = -1);
bool decode_supported(int d, int d_feat);

// Arguments of the backward kernels (gradients of the causal forward).
struct BwdArgs {
  const void *q, *k, *v, *out, *dout;  // [units][n][d] storage type
  const float *den;                    // [units][n], from la_forward_train
  void *dq, *dk, *dv;                  // [units][n][d] storage type
  const float *decay;                  // [H] or null
  int H;
  int64_t n;
  int dqk;    // width of q, k (== d)
  int elu1;   // 1: phi = elu + 1; 0: identity
  // Per-row operands, written by the preparation pass into the workspace:
  // G~ = [dout / den | h hi | h lo | 0 ..] ([units][n][backward_gwidth(d)])
  // and, for elu + 1, K' = phi(k), Q' = phi(q) ([units][n][d]; with the
  // identity map they are k and q themselves).
  void *gt, *kf, *qf;
  // Segmented roles (backward_segments() > 0): segments per role and unit,
  // and their aggregates in the workspace (backward_agg_floats() floats).
  int nseg;
  float *agg;
  // Performer map (else null): K' and Q' are its features ([units][n]
  // [d_feat], in kf, qf), the dq and dk roles write the feature gradients
  // dq', dk' ([units][n][d_feat]) here, and a last pass takes them through
  // the map with omega ([d][d_feat] fp32).
  void *dqf = nullptr, *dkf = nullptr;
  const float *omega = nullptr;
  // Per-position decay (else null): lam = log(gamma) of every position
  // ([units][n] fp32, the layout la_forward_gated takes); decay is null
  // then.
  const float *lam = nullptr;
};
bool backward_supported(int d, int d_feat);
// Sizes the Performer map's backward is built for.
bool backward_performer_supported(int d, int d_feat);
// Enqueue the Performer map's backward (preparation, roles, conversion);
// kf, qf must hold the features already.
hipError_t launch_backward_performer(const BwdArgs &a, int64_t units, int d,
                                     int d_feat, int dtype,
                                     hipStream_t stream);
// Width of a G~ row: d + 2 rounded up to a multiple of 32.
constexpr int backward_gwidth(int d) { return (d + 2 + 31) / 32 * 32; }
// Segments per (role, unit) of the segmented roles (bf16, d = 128), or 0
// where the column-block kernel runs instead; and the floats of their
// aggregates.
int backward_segments(int64_t units, int64_t n, int d, int dtype);
size_t backward_agg_floats(int64_t units, int nseg);
// Enqueue the preparation pass and the role kernels (dq, dk, dv); dtype 0
// fp32, 1 bf16.
hipError_t launch_backward(const BwdArgs &a, int64_t units, int d, int dtype,
                           hipStream_t stream);

}  // namespace la
