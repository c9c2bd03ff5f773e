/*
 * linattn.h -- C ABI of the MI355X (gfx950) causal kernelized linear-attention
 * library (liblinattn.so).
 *
 * What it computes.  Per (batch, head) unit, with a positive feature map phi
 * applied row by row, Q' = phi(Q), K' = phi(K) in R^{n x d'}:
 *
 *   mu_j = g mu_{j-1} + b k'_j^T v_j      (d' x d state)
 *   nu_j = g nu_{j-1} + b k'_j^T          (d' normaliser)
 *   out_j = (q'_j mu_j) / (q'_j . nu_j)   (causal: j reads its own state)
 *
 * with g = b = 1 (no decay) or g = a, b = 1 - a (decay a per head), and zero
 * initial state.  Non-causal: every out_j reads mu_n, nu_n.
 * Sources: "2.2 Linear Attention" (efficient2 page), the feature-mapped Q', K'
 * before eq 6, eq 6, eqs 7-8 (running sums), eq 9 and its causal form, eqs
 * 10-11 (decayed sums); "3.2 Reducing d" (efficient1 page) eqs 22-27 and the
 * remark that both sums are kept and updated as new keys and values arrive;
 * "Linear attention research 2026" page: elu(x) + 1 (Linear Transformer) and
 * exp(x omega - |x|^2/2)/sqrt(m) (Performer random features).
 *
 * Conventions for every entry point.
 *   - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or retains caller memory.
 *   - Row-major, contiguous, no padding.  Prefill tensors are [B][H][n][.],
 *     decode tensors [S][H][.].
 *   - `dtype` is the storage type of q, k, v and out (LA_F32 or LA_BF16).
 *     omega, decay, mu and nu are always fp32.  Arithmetic is fp32 with bf16
 *     (LA_BF16) or fp32 (LA_F32) matrix-core operands.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Calls are asynchronous: they return once the work is enqueued.
 *   - Arguments are validated on the host before anything is enqueued; no
 *     device memory is read for validation.  Decay values and NaN/Inf in the
 *     data are not checked: a must lie in [0, 1].
 *   - Zero sizes (B, H, n, S or rows equal to 0) are a no-op returning LA_OK.
 *   - On error nothing is enqueued (LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED,
 *     LA_ERR_WORKSPACE) or the launch failed (LA_ERR_HIP).  A description of
 *     the last error of the calling thread is kept for la_last_error().
 *   - No C++ exception crosses the ABI.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes */
  LA_ERR_UNSUPPORTED = 2, /* valid request outside the built kernel set      */
  LA_ERR_WORKSPACE = 3,   /* workspace NULL but required                     */
  LA_ERR_HIP = 4,         /* a HIP launch or runtime call failed             */
  LA_ERR_EXCHANGE = 5     /* la_workspace_check: a segment exchange failed   */
} la_status;

typedef enum la_map {
  LA_MAP_IDENTITY = 0,  /* q, k are already features: d_feat wide          */
  LA_MAP_ELU1 = 1,      /* phi(x) = elu(x) + 1 (alpha 1), d_feat == d       */
  LA_MAP_PERFORMER = 2  /* phi(x) = exp(x omega - |x|^2/2)/sqrt(m), d_feat == m */
} la_map;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Layout of the log decay lam = log(gamma) of the gated recurrence (see
 * la_forward_gated).  Values are fp32, device memory. */
typedef enum la_decay_layout {
  LA_LD_CHANNEL = 0,   /* [H][d_feat]: one decay per state row and head     */
  LA_LD_POSITION = 1,  /* [B][H][n] (decode: [S][H]): one per position      */
  LA_LD_BOTH = 2       /* [B][H][n][d_feat] (decode: [S][H][d_feat])        */
} la_decay_layout;

/*
 * la_featmap -- phi applied row by row: x [rows][d] -> x_feat [rows][d_feat].
 *   "Linear attention research 2026" page, Performer and Linear Transformer
 *   sections; Q' = phi(Q) of "2.2 Linear Attention".
 *   x      : device, in_dt, [rows][d]
 *   x_feat : device, out_dt, [rows][d_feat] with d_feat = m (PERFORMER) or d
 *   omega  : device fp32 [d][m] for PERFORMER (one projection shared by all
 *            rows); ignored (may be NULL) otherwise
 *   m      : feature count for PERFORMER; ignored otherwise
 *   Supported: d in {16, 32, 64, 128}; m a multiple of 16 in [16, 256].
 */
la_status la_featmap(const void *x, void *x_feat, const float *omega,
                     int64_t rows, int d, int m, la_map map, la_dtype in_dt,
                     la_dtype out_dt, void *stream);

/*
 * la_forward_workspace_bytes -- device workspace la_forward needs for these
 * sizes (0 when none).  Pure host function, never fails: returns 0 for
 * arguments la_forward would reject.
 */
size_t la_forward_workspace_bytes(int B, int H, int64_t n, int d, int d_feat,
                                  la_map map, la_dtype dtype, int causal);

/*
 * la_forward -- causal (causal = 1) or non-causal (causal = 0) kernelized
 * attention over B*H independent units, state starting at zero.
 *   "2.2 Linear Attention" eqs 7-11 and the causal form of eq 9; non-causal
 *   is eq 9 with mu_n, nu_n (eq 6; "3.2 Reducing d" eq 27).
 *   q, k     : device, dtype, [B][H][n][d] (ELU1, PERFORMER) or
 *              [B][H][n][d_feat] (IDENTITY: already feature-mapped)
 *   v, out   : device, dtype, [B][H][n][d]; out may not alias q, k or v
 *   d_feat   : d for ELU1, m for PERFORMER, the feature width for IDENTITY
 *   omega    : device fp32 [d][d_feat] for PERFORMER, else ignored
 *   decay    : device fp32 [H], one a per head, or NULL for eqs 7-8
 *   workspace: device, at least la_forward_workspace_bytes(...) bytes; NULL
 *              allowed only when that is 0.  Whenever a call uses a
 *              workspace, its first 65792 bytes are a synchronisation area:
 *              calls whose sequence is split into segments (B * H < 512)
 *              use it, and no call writes anything else there.  It must be
 *              zero before the first call that uses the workspace (zero the
 *              whole workspace once at allocation) and every call leaves it
 *              zero, so one workspace can serve calls of any sizes.  The
 *              rest is scratch.  Calls that may run concurrently (different
 *              streams) must not share a workspace.
 *              What a violation does: causal segments of a unit exchange
 *              their partial sums through flags in that area.  A flag left
 *              set (area not zeroed, or a concurrent call on another stream)
 *              lets a segment read a partial sum before it is written: its
 *              outputs are then wrong.  A ticket found out of range marks
 *              the workspace's status word "corrupt"; a wait that never sees
 *              its flag gives up after a bounded number of polls (about a
 *              second or more by default), marks the status word "timeout"
 *              and writes NaN to every output that depended on the missing
 *              sum.  The kernel always finishes.  la_workspace_check reports
 *              and clears that status word.
 *   Supported: d in {16, 32, 64, 128}; d_feat in {16, 32, 64, 128, 256}.
 *   No epsilon is added to the denominator: with IDENTITY features whose
 *   q'.nu is zero the output is inf/nan (IEEE).
 */
la_status la_forward(const void *q, const void *k, const void *v, void *out,
                     int B, int H, int64_t n, int d, int d_feat, la_map map,
                     const float *omega, const float *decay, int causal,
                     la_dtype dtype, void *workspace, void *stream);

/*
 * la_forward_state -- la_forward that also hands out the state after the
 * last position of every unit, the sums the decode step continues from:
 * mu_n = sum_j w_j k'_j^T v_j and nu_n = sum_j w_j k'_j ("2.2 Linear
 * Attention" eqs 7-8, or eqs 10-11 with decay; "3.2 Reducing d", remark
 * after eq 27: the two sums are kept and updated as tokens arrive).
 *   All arguments as la_forward, plus:
 *   mu_out : device fp32 [B][H][d_feat][d], written (the decode step's mu)
 *   nu_out : device fp32 [B][H][d_feat], written (the decode step's nu)
 *   Both required (LA_ERR_INVALID_ARG if either is NULL).  With n == 0 they
 *   are set to zero.  The state is fp32 as accumulated by the kernel; with
 *   causal = 0 it is the total every row was read against (the same mu_n).
 */
la_status la_forward_state(const void *q, const void *k, const void *v,
                           void *out, int B, int H, int64_t n, int d,
                           int d_feat, la_map map, const float *omega,
                           const float *decay, int causal, la_dtype dtype,
                           void *workspace, float *mu_out, float *nu_out,
                           void *stream);

/*
 * la_forward_noalloc -- la_forward that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Its scratch is a static device array of the library, 32 MiB, one copy per
 * GPU, held until the process ends; the first call on a device looks it up
 * and clears its synchronisation area with a fill kernel on `stream`.
 *   Arguments, layouts, support and errors as la_forward, without
 *   `workspace`.  The stream must belong to the current device.  When a
 *   call's segment partial sums would not fit in the scratch, it splits the
 *   sequence into fewer segments (results within the same tolerance).  The
 *   Performer map with fp32 storage (or sizes the fused map is not built
 *   for), which needs n-sized feature buffers, is rejected with
 *   LA_ERR_UNSUPPORTED.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (different streams, or different threads) race and must be
 *   serialised by the caller.  Exchange failures show as NaN outputs (there
 *   is no workspace to check).
 */
la_status la_forward_noalloc(const void *q, const void *k, const void *v,
                             void *out, int B, int H, int64_t n, int d,
                             int d_feat, la_map map, const float *omega,
                             const float *decay, int causal, la_dtype dtype,
                             void *stream);

/*
 * la_forward_train -- the causal la_forward that also writes each row's
 * denominator den_j = q'_j . nu_j, as the backward pass needs it ("2.2
 * Linear Attention" eq 9, causal form: out_j = q'_j mu_j / den_j).
 *   All arguments as la_forward (causal), plus
 *   den : device fp32 [B][H][n], written; LA_ERR_INVALID_ARG if NULL.
 */
la_status la_forward_train(const void *q, const void *k, const void *v,
                           void *out, float *den, int B, int H, int64_t n,
                           int d, int d_feat, la_map map, const float *omega,
                           const float *decay, la_dtype dtype, void *workspace,
                           void *stream);

/*
 * la_backward -- gradients of sum(out * dout) with respect to q, k and v for
 * the causal forward (eqs 7-11 with the feature map), for training through
 * it ("Linear attention research 2026" page, closing section: parallel
 * training of the recurrent forms).  With G_j = [dout_j / den_j |
 * -(dout_j . out_j) / den_j] and w_ij the weights of eqs 7-8 / 10-11:
 *   dq'_i = sum_{j<=i} w_ij (G_i . [v_j|1]) k'_j,
 *   dk'_j = sum_{i>=j} w_ij (G_i . [v_j|1]) q'_i,
 *   dv_j  = sum_{i>=j} w_ij (q'_i . k'_j) dout_i / den_i,
 * then through the feature map (elu + 1: times 1 for x > 0, e^x else;
 * Performer, "Linear attention research 2026" page, Performer section:
 * d phi_r / d x = phi_r(x) (omega_r - x), so dx = (dx' * phi(x)) omega^T -
 * x (dx' . phi(x)), where for the queries dq' . phi(q) = 0 exactly, each
 * output being unchanged by a scaling of its q', and that term is dropped).
 *   q, k, v, out, dout: device, dtype, [B][H][n][d] (out and den as
 *                       la_forward_train wrote them for these q, k, v)
 *   den   : device fp32 [B][H][n]
 *   dq, dk, dv: device, dtype, [B][H][n][d], written (may not alias inputs)
 *   map   : LA_MAP_ELU1, LA_MAP_IDENTITY or LA_MAP_PERFORMER
 *   omega : LA_MAP_PERFORMER: device fp32 [d][d_feat], the forward's;
 *           LA_ERR_INVALID_ARG if NULL; not differentiated.  Else ignored.
 *   decay : device fp32 [H] or NULL, as la_forward
 *   workspace: device, at least la_backward_workspace_bytes(...) bytes, no
 *           initial contents needed; LA_ERR_WORKSPACE if NULL.  Calls that
 *           share one workspace must be ordered (one stream).
 *   Supported: ELU1, IDENTITY: d == d_feat in {16, 32, 64, 128};
 *              PERFORMER: d in {32, 64, 128}, d_feat in {32, 64, 128, 256},
 *              d * d_feat <= 16384.  Other sizes: LA_ERR_UNSUPPORTED.
 */
la_status la_backward(const void *q, const void *k, const void *v,
                      const void *out, const float *den, const void *dout,
                      void *dq, void *dk, void *dv, int B, int H, int64_t n,
                      int d, int d_feat, la_map map, const float *omega,
                      const float *decay, la_dtype dtype, void *workspace,
                      void *stream);

/*
 * la_backward_workspace_bytes -- device workspace la_backward needs for
 * these sizes: per row, the prepared G row (d + 2 values padded to a
 * multiple of 32) and, for LA_MAP_ELU1, the features phi(k) and phi(q), all
 * in dtype; for LA_MAP_PERFORMER the features phi(k), phi(q) (d_feat values
 * each, dtype) and the feature gradients dq', dk' (d_feat values each,
 * fp32).  Pure host function; 0 for arguments la_backward would reject and
 * for empty sizes.
 */
size_t la_backward_workspace_bytes(int B, int H, int64_t n, int d, int d_feat,
                                   la_map map, la_dtype dtype);

/*
 * la_forward_gated_workspace_bytes -- device workspace la_forward_gated
 * needs for these sizes and this decay layout (0 when none).  For
 * LA_LD_POSITION it equals la_forward_workspace_bytes of the same sizes; for
 * a decay per state row it covers the segment aggregates (and Q', K' for
 * PERFORMER).  Pure host function, never fails: returns 0 for arguments
 * la_forward_gated would reject.
 */
size_t la_forward_gated_workspace_bytes(int B, int H, int64_t n, int d,
                                        int d_feat, la_map map,
                                        la_decay_layout layout, la_dtype dtype,
                                        int causal);

/*
 * la_forward_gated -- la_forward / la_forward_state with a decay that
 * varies by position and/or state row: gamma = exp(lam) replaces a in
 * eqs 10-11, row f of the state at position j decaying by gamma_j[f],
 *   mu_j[f] = gamma_j[f] mu_{j-1}[f] + (1 - gamma_j[f]) k'_j[f] v_j,
 *   nu_j[f] = gamma_j[f] nu_{j-1}[f] + (1 - gamma_j[f]) k'_j[f],
 * read out as in la_forward.  One decay per row (LA_LD_CHANNEL) is the
 * diagonal A of "2.3 State-Space Models" eqs 21-25; one per position
 * (LA_LD_POSITION) is the input-dependent decay of Mamba's selective step,
 * dA = exp(A delta_t) ("Linear attention research 2026" page), and
 * LA_LD_BOTH is that decay per row.  1 - gamma is the zero-order-hold input
 * weight of the discretised update of "2.3 State-Space Models" eq 14, up to
 * a constant that cancels in the ratio.
 *   All arguments as la_forward, with
 *   log_decay: device fp32 lam = log(gamma) in `layout`; values <= 0
 *              (decays in (0, 1]) are expected and not checked; -inf gives
 *              gamma = 0 (the state row restarts at that position).
 *   layout   : LA_LD_POSITION ([B][H][n]), LA_LD_CHANNEL ([H][d_feat]) or
 *              LA_LD_BOTH ([B][H][n][d_feat]).  With a decay per row, the
 *              products of queries and keys inside a 16-position chunk
 *              floor each step's decay at 2^-32: a step that decays more
 *              forgets what came before it inside its chunk to within
 *              2.3e-10 of its weight instead of fully; across chunks and in
 *              the state the decay is exact.
 *   mu_out, nu_out: optional (both or neither), as la_forward_state.
 *   workspace: la_forward_gated_workspace_bytes(...) of the same sizes and
 *              layout, with the synchronisation area of la_forward zero
 *              (the per-row path never writes it).
 */
la_status la_forward_gated(const void *q, const void *k, const void *v,
                           void *out, int B, int H, int64_t n, int d,
                           int d_feat, la_map map, const float *omega,
                           const float *log_decay, la_decay_layout layout,
                           int causal, la_dtype dtype, void *workspace,
                           float *mu_out, float *nu_out, void *stream);

/*
 * la_forward_gated_train -- the causal la_forward_gated with one decay per
 * position that also writes each row's denominator, for la_backward_gated
 * (as la_forward_train does for la_backward).
 *   All arguments as la_forward_gated (causal, no handed-out state), plus
 *   den   : device fp32 [B][H][n], written; LA_ERR_INVALID_ARG if NULL.
 *   layout: LA_LD_POSITION only; the other layouts return
 *           LA_ERR_UNSUPPORTED.
 *   workspace: la_forward_gated_workspace_bytes(...) with LA_LD_POSITION
 *           and causal = 1, synchronisation area zero as for la_forward.
 */
la_status la_forward_gated_train(const void *q, const void *k, const void *v,
                                 void *out, float *den, int B, int H,
                                 int64_t n, int d, int d_feat, la_map map,
                                 const float *omega, const float *log_decay,
                                 la_decay_layout layout, la_dtype dtype,
                                 void *workspace, void *stream);

/*
 * la_backward_gated -- la_backward for the causal forward with one decay
 * per position (la_forward_gated, LA_LD_POSITION: the input-dependent decay
 * of Mamba's selective step, "Linear attention research 2026" page; the
 * recurrence of la_forward_gated).  The weights of la_backward become
 *   w_ij = (1 - gamma_j) prod_{p=j+1..i} gamma_p   (j <= i),
 * and the decay itself is an input that is not differentiated.
 *   All arguments as la_backward, with out and den from
 *   la_forward_gated_train, and
 *   log_decay: device fp32 lam = log(gamma), [B][H][n], as the forward's;
 *              LA_ERR_INVALID_ARG if NULL for non-empty sizes.  Values
 *              below -104 act as -104 (gamma = 0 in fp32 either way).
 *   layout   : LA_LD_POSITION; the other layouts return LA_ERR_UNSUPPORTED.
 *   workspace: device, at least la_backward_gated_workspace_bytes(...).
 *   Supported: the sizes la_backward supports, for all three maps.
 */
la_status la_backward_gated(const void *q, const void *k, const void *v,
                            const void *out, const float *den,
                            const void *dout, void *dq, void *dk, void *dv,
                            int B, int H, int64_t n, int d, int d_feat,
                            la_map map, const float *omega,
                            const float *log_decay, la_decay_layout layout,
                            la_dtype dtype, void *workspace, void *stream);

/*
 * la_backward_gated_workspace_bytes -- device workspace la_backward_gated
 * needs: that of la_backward for the same sizes and map (the segment state
 * sums carry each segment's sum of log2 gamma in space la_backward
 * reserves).
 * Pure host function; 0 for arguments la_backward_gated would reject and
 * for empty sizes.
 */
size_t la_backward_gated_workspace_bytes(int B, int H, int64_t n, int d,
                                         int d_feat, la_map map,
                                         la_dtype dtype);

/*
 * la_decode_step_gated -- la_decode_step with a decay per state row and/or
 * per unit: row f of unit u decays by gamma = exp(lam) with input weight
 * 1 - gamma (the diagonal A of "2.3 State-Space Models" eqs 21-25, and
 * Mamba's input-dependent decay).
 *   All arguments as la_decode_step, with
 *   log_decay: device fp32 lam, [H][d_feat] (LA_LD_CHANNEL), [S][H]
 *              (LA_LD_POSITION: this step's decay per unit) or
 *              [S][H][d_feat] (LA_LD_BOTH); LA_ERR_INVALID_ARG if NULL.
 */
la_status la_decode_step_gated(float *mu, float *nu, const void *q,
                               const void *k, const void *v, void *out, int S,
                               int H, int d, int d_feat, la_map map,
                               const float *omega, const float *log_decay,
                               la_decay_layout layout, la_dtype dtype,
                               void *stream);

/*
 * la_decode_step -- one autoregressive step per (sequence, head) unit: the
 * running sums are updated in place by the new (k, v) and the new token's
 * output is read out from the UPDATED sums (it attends to itself).
 *   "3.2 Reducing d", remark after eq 27 (keep both sums, update them as new
 *   keys and values arrive); "2.2 Linear Attention" eqs 7-8 / 10-11 and the
 *   causal form of eq 9.
 *   mu    : device fp32 [S][H][d_feat][d], read and overwritten
 *   nu    : device fp32 [S][H][d_feat], read and overwritten
 *   q, k  : device, dtype, [S][H][d] (or [S][H][d_feat] for IDENTITY)
 *   v, out: device, dtype, [S][H][d]
 *   omega : device fp32 [d][d_feat] for PERFORMER, else ignored
 *   decay : device fp32 [H] or NULL (no decay: mu += k'^T v, nu += k')
 *   Supported: d in {16, 32, 64, 128}; d_feat in {16, 32, 64, 128, 256}.
 */
la_status la_decode_step(float *mu, float *nu, const void *q, const void *k,
                         const void *v, void *out, int S, int H, int d,
                         int d_feat, la_map map, const float *omega,
                         const float *decay, la_dtype dtype, void *stream);

/*
 * la_workspace_check -- whether any call that used this workspace since the
 * last check had a segment exchange fail (see la_forward's workspace notes):
 * LA_OK if none, LA_ERR_EXCHANGE otherwise (la_last_error says which kind;
 * the status is then cleared).  It waits for the work enqueued on `stream`,
 * then reads 4 bytes of the workspace: a synchronising diagnostic, not for a
 * hot loop.  workspace: device, a la_forward workspace (at least 65792
 * bytes); LA_ERR_INVALID_ARG if NULL.
 */
la_status la_workspace_check(void *workspace, void *stream);

/*
 * la_set_exchange_spin_limit -- diagnostics: polls a segment's wait for
 * another segment's partial sum makes before giving up (0 restores the
 * default, about 2^22 polls).  Process-wide; applies to calls enqueued
 * afterwards.  A small limit lets a test force the failure path of
 * la_workspace_check while every kernel still ends normally.
 */
void la_set_exchange_spin_limit(unsigned spins);

/* Static description of a status code (never NULL). */
const char *la_status_str(la_status status);

/* Description of the calling thread's last error ("" if none). */
const char *la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
