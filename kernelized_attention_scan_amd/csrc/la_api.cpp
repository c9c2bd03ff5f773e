// C ABI of liblinattn.so: argument validation, workspace planning and kernel
// dispatch.  Validation is pure host code that runs before any HIP call, so
// invalid requests never touch a device.  See include/linattn.h for the
// contract of every entry point.
#include "linattn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "la_internal.h"

namespace {

thread_local std::string g_last_error;

// Polls of an exchange wait before it gives up (la_set_exchange_spin_limit).
std::atomic<unsigned> g_spin_limit{la::kDefaultSpinLimit};

la_status fail(la_status st, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
la_status fail(la_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

la_status ok() {
  g_last_error.clear();
  return LA_OK;
}

la_status hip_fail(hipError_t e, const char *what) {
  return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_map(int m) { return m == LA_MAP_IDENTITY || m == LA_MAP_ELU1 || m == LA_MAP_PERFORMER; }
bool valid_dtype(int t) { return t == LA_F32 || t == LA_BF16; }
bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_feat(int f) {
  return f == 16 || f == 32 || f == 64 || f == 128 || f == 256;
}
size_t elem_size(int t) { return t == LA_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Sequence split of the fused forward: about la::kCUs workgroups in total,
// at most la::kMaxSegments segments of whole chunks per (batch, head) unit.  A unit
// gets several segments only when there are fewer units than that.  No
// split needs its workgroups to be resident at once: causal segments are
// numbered in start order, non-causal ones run as two launches.
constexpr int64_t kMaxSegments = la::kMaxSegments;

struct FwdPlan {
  const la::FwdOps *ops = nullptr;
  int64_t seg_len = 0;
  int nseg = 0;
  bool need_states = false;
  bool fused_performer = false;  // Performer map applied inside the forward
  size_t feat_bytes = 0;    // one of Q', K' (unfused PERFORMER only)
  size_t sync_bytes = 0;    // synchronisation area
  size_t agg_bytes = 0;     // segment aggregates
  // synchronisation area + segment aggregates + each segment's sum of log2
  // decay (used with per-position decay; reserved always, so a workspace's
  // size does not depend on the kind of decay)
  size_t state_bytes = 0;
  // Q', K' start after the aggregates, and never below the fixed
  // synchronisation area even when this call has no segments: a workspace
  // shared with segmented calls keeps that area zero between calls, so no
  // other data may ever be written there.
  size_t feat_offset() const {
    return state_bytes > 0 ? state_bytes : la::kSyncBytes;
  }
  size_t total() const {
    return feat_bytes > 0 ? feat_offset() + 2 * feat_bytes : state_bytes;
  }
};

// Validates la_forward's sizes and enums (not pointers) and fills the plan.
// A non-zero state_cap bounds the synchronisation area plus the segment
// aggregates: the split then takes fewer segments per unit until they fit.
// decay: 0 none, 1 one value per head, 2 one per position.
la_status plan_forward(int B, int H, int64_t n, int d, int d_feat, int map,
                       int dtype, int causal, int decay, FwdPlan *p,
                       size_t state_cap = 0) {
  if (B < 0 || H < 0 || n < 0)
    return fail(LA_ERR_INVALID_ARG, "negative size: B=%d H=%d n=%lld", B, H,
                static_cast<long long>(n));
  if (!valid_map(map)) return fail(LA_ERR_INVALID_ARG, "unknown map %d", map);
  if (!valid_dtype(dtype)) return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (causal != 0 && causal != 1)
    return fail(LA_ERR_INVALID_ARG, "causal must be 0 or 1, got %d", causal);
  if (d <= 0 || d_feat <= 0)
    return fail(LA_ERR_INVALID_ARG, "non-positive d=%d d_feat=%d", d, d_feat);
  if (map == LA_MAP_ELU1 && d_feat != d)
    return fail(LA_ERR_INVALID_ARG, "ELU1 needs d_feat == d (got %d, %d)", d_feat, d);
  if (!supported_d(d) || !supported_feat(d_feat))
    return fail(LA_ERR_UNSUPPORTED, "unsupported d=%d d_feat=%d", d, d_feat);
  // The Performer map is fused into the forward where an instance is built
  // for these sizes (with its decayed variant, so the workspace does not
  // depend on decay); otherwise q', k' go through the workspace.
  if (map == LA_MAP_PERFORMER && dtype == LA_BF16) {
    const la::FwdOps *pf = la::fwd_ops_bf16_performer(d, d_feat);
    if (pf && pf->decay_ok && pf->sel_ok) {
      p->ops = pf;
      p->fused_performer = true;
    }
  }
  if (!p->fused_performer)
    p->ops = dtype == LA_BF16 ? la::fwd_ops_bf16(d, d_feat) : la::fwd_ops_f32(d, d_feat);
  if (!p->ops || (decay == 1 && !p->ops->decay_ok) ||
      (decay == 2 && !p->ops->sel_ok))
    return fail(LA_ERR_UNSUPPORTED, "no %s%s kernel for d=%d d_feat=%d (LDS)",
                dtype == LA_BF16 ? "bf16" : "fp32",
                decay == 1 ? " decayed" : decay == 2 ? " gated" : "", d,
                d_feat);
  const int64_t units = static_cast<int64_t>(B) * H;
  if (units == 0 || n == 0) return LA_OK;
  if (units > (int64_t{1} << 30) || n > (int64_t{1} << 40) ||
      units * n > (int64_t{1} << 46))
    return fail(LA_ERR_UNSUPPORTED, "sizes too large");
  const int64_t C = p->ops->C;
  const int64_t nchunks = (n + C - 1) / C;
  // about one workgroup per compute unit: measured faster than filling a
  // second workgroup slot per CU with shorter segments (the chain phase 1 ->
  // exchange -> phase 2 is shorter with fewer, longer segments)
  // (with a value split each unit is vsplit computations of its own)
  const int64_t vunits = units * p->ops->vsplit;
  const int64_t target = la::kCUs;
  int64_t per_unit = (target + vunits - 1) / vunits;
  if (per_unit > kMaxSegments) per_unit = kMaxSegments;
  if (per_unit < 1) per_unit = 1;
  if (per_unit > nchunks) per_unit = nchunks;
  if (state_cap > 0) {
    const size_t slot = static_cast<size_t>(p->ops->slot_floats) * sizeof(float);
    auto need = [&](int64_t k) {
      return la::kSyncBytes + align256(static_cast<size_t>(vunits) * k * slot) +
             align256(static_cast<size_t>(vunits) * k * sizeof(float));
    };
    while (per_unit > 1 && need(per_unit) > state_cap) --per_unit;
  }
  const int64_t cps = (nchunks + per_unit - 1) / per_unit;
  p->seg_len = cps * C;
  p->nseg = static_cast<int>((n + p->seg_len - 1) / p->seg_len);
  if (vunits * p->nseg > (int64_t{1} << 31) - 1)
    return fail(LA_ERR_UNSUPPORTED, "too many workgroups");
  p->need_states = p->nseg > 1;
  if (p->need_states && vunits >= la::kMaxTargetGroups)
    return fail(LA_ERR_HIP, "internal: segmented split for %lld units",
                static_cast<long long>(vunits));
  p->sync_bytes = p->need_states ? la::kSyncBytes : 0;
  p->agg_bytes = p->need_states
                     ? align256(static_cast<size_t>(vunits) * p->nseg *
                                p->ops->slot_floats * sizeof(float))
                     : 0;
  p->state_bytes =
      p->need_states
          ? p->sync_bytes + p->agg_bytes +
                align256(static_cast<size_t>(vunits) * p->nseg * sizeof(float))
          : 0;
  p->feat_bytes = map == LA_MAP_PERFORMER && !p->fused_performer
                      ? align256(static_cast<size_t>(units * n) * d_feat *
                                 elem_size(dtype))
                      : 0;
  return LA_OK;
}

// Plan of the forward with a decay per state row: segments of whole
// 16-row chunks, their aggregates after the synchronisation area (which it
// never writes, so a workspace shared with la_forward keeps that area zero),
// then Q', K' for the Performer map.
struct RowPlan {
  const la::RowOps *ops = nullptr;
  int64_t seg_len = 0;
  int nseg = 0;
  size_t agg_bytes = 0;   // [units][nseg + 1] aggregate slots
  size_t feat_bytes = 0;  // one of Q', K' (PERFORMER)
  size_t feat_offset() const { return la::kSyncBytes + agg_bytes; }
  size_t total() const {
    return agg_bytes + feat_bytes > 0 ? feat_offset() + 2 * feat_bytes : 0;
  }
};

la_status plan_rows(int B, int H, int64_t n, int d, int d_feat, int map,
                    int dtype, int causal, RowPlan *p) {
  if (B < 0 || H < 0 || n < 0)
    return fail(LA_ERR_INVALID_ARG, "negative size: B=%d H=%d n=%lld", B, H,
                static_cast<long long>(n));
  if (!valid_map(map)) return fail(LA_ERR_INVALID_ARG, "unknown map %d", map);
  if (!valid_dtype(dtype)) return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (causal != 0 && causal != 1)
    return fail(LA_ERR_INVALID_ARG, "causal must be 0 or 1, got %d", causal);
  if (d <= 0 || d_feat <= 0)
    return fail(LA_ERR_INVALID_ARG, "non-positive d=%d d_feat=%d", d, d_feat);
  if (map == LA_MAP_ELU1 && d_feat != d)
    return fail(LA_ERR_INVALID_ARG, "ELU1 needs d_feat == d (got %d, %d)", d_feat, d);
  if (!supported_d(d) || !supported_feat(d_feat))
    return fail(LA_ERR_UNSUPPORTED, "unsupported d=%d d_feat=%d", d, d_feat);
  p->ops = la::row_ops(d, d_feat, dtype == LA_BF16 ? 1 : 0);
  if (!p->ops)
    return fail(LA_ERR_UNSUPPORTED, "no per-row decay kernel for d=%d d_feat=%d",
                d, d_feat);
  const int64_t units = static_cast<int64_t>(B) * H;
  if (units == 0 || n == 0) return LA_OK;
  if (units > (int64_t{1} << 30) || n > (int64_t{1} << 40) ||
      units * n > (int64_t{1} << 46))
    return fail(LA_ERR_UNSUPPORTED, "sizes too large");
  const int64_t C = la::kRowChunk;
  const int64_t nch = (n + C - 1) / C;
  const int64_t k = la::row_segments(units, n);
  const int64_t cps = (nch + k - 1) / k;
  p->seg_len = cps * C;
  p->nseg = static_cast<int>((n + p->seg_len - 1) / p->seg_len);
  if (units * p->nseg > (int64_t{1} << 31) - 1 ||
      units * ((p->ops->slot_floats + 255) / 256) > (int64_t{1} << 31) - 1)
    return fail(LA_ERR_UNSUPPORTED, "too many workgroups");
  p->agg_bytes = !causal || p->nseg > 1
                     ? align256(static_cast<size_t>(units) * (p->nseg + 1) *
                                p->ops->slot_floats * sizeof(float))
                     : 0;
  p->feat_bytes = map == LA_MAP_PERFORMER
                      ? align256(static_cast<size_t>(units * n) * d_feat *
                                 elem_size(dtype))
                      : 0;
  return LA_OK;
}

}  // namespace

// la_forward and la_forward_state; mu_out / nu_out (both or neither) receive
// the state after the last position.
// workspace_cap != 0: the workspace holds only that many bytes (the
// allocation-free entry point), so the plan fits its split into it and
// rejects the unfused Performer map, whose features need n-sized buffers.
// log_decay (per-position decay, [B][H][n]) replaces decay when given.
static la_status forward_impl(const void *q, const void *k, const void *v, void *out,
                       int B, int H, int64_t n, int d, int d_feat, int map,
                       const float *omega, const float *decay, int causal,
                       int dtype, void *workspace, float *mu_out, float *nu_out,
                       void *stream, size_t workspace_cap = 0,
                       const float *log_decay = nullptr,
                       float *den_out = nullptr) {
  try {
    FwdPlan p;
    const int dkind = log_decay ? 2 : decay ? 1 : 0;
    const la_status st = plan_forward(B, H, n, d, d_feat, map, dtype, causal,
                                      dkind, &p, workspace_cap);
    if (st != LA_OK) return st;
    if (workspace_cap > 0 && p.total() > workspace_cap)
      return fail(LA_ERR_UNSUPPORTED, "workspace of %zu bytes needed, %zu held",
                  p.total(), workspace_cap);
    const int64_t units = static_cast<int64_t>(B) * H;
    if (units == 0) return ok();
    if (n == 0) {  // no positions: the handed-out state is zero
      if (!mu_out) return ok();
      hipStream_t s = static_cast<hipStream_t>(stream);
      hipError_t e = la::launch_fill_zero(mu_out, units * d_feat * d, s);
      if (e == hipSuccess) e = la::launch_fill_zero(nu_out, units * d_feat, s);
      if (e != hipSuccess) return hip_fail(e, "la_forward_state zero state");
      return ok();
    }
    if (!q || !k || !v || !out)
      return fail(LA_ERR_INVALID_ARG, "null q, k, v or out");
    if (map == LA_MAP_PERFORMER && !omega)
      return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
    if ((mu_out == nullptr) != (nu_out == nullptr))
      return fail(LA_ERR_INVALID_ARG, "mu_out and nu_out go together");
    if (p.total() > 0 && !workspace)
      return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required", p.total());
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const void *qf = q, *kf = k;
    if (map == LA_MAP_PERFORMER && !p.fused_performer) {
      // Q', K' into the workspace, then the identity-map forward over them.
      unsigned char *fq = ws + p.feat_offset(), *fk = fq + p.feat_bytes;
      hipError_t e = la::launch_featmap_performer(q, fq, omega, units * n, d,
                                                  d_feat, dtype, dtype, s);
      if (e == hipSuccess)
        e = la::launch_featmap_performer(k, fk, omega, units * n, d, d_feat,
                                         dtype, dtype, s);
      if (e != hipSuccess) return hip_fail(e, "la_forward feature map");
      qf = fq;
      kf = fk;
    }
    la::FwdArgs a;
    a.q = qf;
    a.k = kf;
    a.v = v;
    a.out = out;
    a.decay = decay;
    a.sync = p.need_states ? reinterpret_cast<unsigned *>(ws) : nullptr;
    a.states = p.need_states ? reinterpret_cast<float *>(ws + p.sync_bytes)
                             : nullptr;
    a.seg_log = p.need_states ? reinterpret_cast<float *>(
                                    ws + p.sync_bytes + p.agg_bytes)
                              : nullptr;
    a.log_decay = log_decay;
    a.den_out = den_out;
    a.H = H;
    a.n = n;
    a.seg_len = p.seg_len;
    a.nseg = p.nseg;
    a.elu1 = map == LA_MAP_ELU1;
    a.omega = p.fused_performer ? omega : nullptr;
    a.mu_out = mu_out;
    a.nu_out = nu_out;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    const hipError_t e = p.ops->run(a, units, causal, s);
    if (e != hipSuccess) return hip_fail(e, "la_forward launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_forward");
  }
}

// la_forward_gated with a decay per state row (lam [H][d_feat], or
// [B][H][n][d_feat] with per_position).
static la_status forward_rows_impl(const void *q, const void *k, const void *v,
                                   void *out, int B, int H, int64_t n, int d,
                                   int d_feat, int map, const float *omega,
                                   const float *log_decay, int per_position,
                                   int causal, int dtype, void *workspace,
                                   float *mu_out, float *nu_out, void *stream) {
  try {
    RowPlan p;
    const la_status st =
        plan_rows(B, H, n, d, d_feat, map, dtype, causal, &p);
    if (st != LA_OK) return st;
    const int64_t units = static_cast<int64_t>(B) * H;
    if (units == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 0) {  // no positions: the handed-out state is zero
      if (!mu_out) return ok();
      hipError_t e = la::launch_fill_zero(mu_out, units * d_feat * d, s);
      if (e == hipSuccess) e = la::launch_fill_zero(nu_out, units * d_feat, s);
      if (e != hipSuccess) return hip_fail(e, "la_forward_gated zero state");
      return ok();
    }
    if (!q || !k || !v || !out)
      return fail(LA_ERR_INVALID_ARG, "null q, k, v or out");
    if (map == LA_MAP_PERFORMER && !omega)
      return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
    if (p.total() > 0 && !workspace)
      return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes required", p.total());
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const void *qf = q, *kf = k;
    if (map == LA_MAP_PERFORMER) {
      unsigned char *fq = ws + p.feat_offset(), *fk = fq + p.feat_bytes;
      hipError_t e = la::launch_featmap_performer(q, fq, omega, units * n, d,
                                                  d_feat, dtype, dtype, s);
      if (e == hipSuccess)
        e = la::launch_featmap_performer(k, fk, omega, units * n, d, d_feat,
                                         dtype, dtype, s);
      if (e != hipSuccess) return hip_fail(e, "la_forward_gated feature map");
      qf = fq;
      kf = fk;
    }
    la::RowArgs a;
    a.q = qf;
    a.k = kf;
    a.v = v;
    a.out = out;
    a.lam = log_decay;
    a.per_position = per_position;
    a.H = H;
    a.n = n;
    a.seg_len = p.seg_len;
    a.nseg = p.nseg;
    a.elu1 = map == LA_MAP_ELU1;
    a.skip_last = 0;
    a.agg = p.agg_bytes > 0 ? reinterpret_cast<float *>(ws + la::kSyncBytes)
                            : nullptr;
    a.mu_out = mu_out;
    a.nu_out = nu_out;
    const hipError_t e = p.ops->run(a, units, causal, s);
    if (e != hipSuccess) return hip_fail(e, "la_forward_gated launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_forward_gated");
  }
}

// ---------------------------------------------------------------------------
// Allocation-free forward: its workspace is this file-scope device array,
// one copy per GPU, held until the process ends.  In host code `scratch` is
// only a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t{32} << 20;
static_assert(kScratchBytes > la::kSyncBytes, "scratch holds the sync area");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// This device's copy of `scratch`.  The first call on a device looks the
// address up and zeroes the synchronisation area at its start with a fill
// kernel on the caller's stream (every forward leaves that area zero
// again); later calls reuse the address.
la_status device_scratch(hipStream_t s, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "la_forward_noalloc device");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(LA_ERR_UNSUPPORTED, "la_forward_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "la_forward_noalloc scratch address");
    e = la::launch_fill_zero(static_cast<float *>(ptr),
                             static_cast<int64_t>(la::kSyncBytes / sizeof(float)),
                             s);
    if (e != hipSuccess) return hip_fail(e, "la_forward_noalloc scratch clear");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}
}  // namespace

extern "C" {

const char *la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_HIP: return "LA_ERR_HIP";
    case LA_ERR_EXCHANGE: return "LA_ERR_EXCHANGE";
  }
  return "LA_ERR_UNKNOWN";
}

const char *la_last_error(void) { return g_last_error.c_str(); }

la_status la_featmap(const void *x, void *x_feat, const float *omega,
                     int64_t rows, int d, int m, la_map map, la_dtype in_dt,
                     la_dtype out_dt, void *stream) {
  try {
    if (rows < 0) return fail(LA_ERR_INVALID_ARG, "negative rows");
    if (!valid_map(map)) return fail(LA_ERR_INVALID_ARG, "unknown map %d", map);
    if (!valid_dtype(in_dt) || !valid_dtype(out_dt))
      return fail(LA_ERR_INVALID_ARG, "unknown dtype");
    if (d <= 0) return fail(LA_ERR_INVALID_ARG, "non-positive d=%d", d);
    if (map == LA_MAP_PERFORMER && m <= 0)
      return fail(LA_ERR_INVALID_ARG, "non-positive m=%d", m);
    if (!supported_d(d)) return fail(LA_ERR_UNSUPPORTED, "unsupported d=%d", d);
    if (map == LA_MAP_PERFORMER && (m % 16 != 0 || m > 256))
      return fail(LA_ERR_UNSUPPORTED, "unsupported m=%d (multiple of 16, <= 256)", m);
    if (rows == 0) return ok();
    if (!x || !x_feat) return fail(LA_ERR_INVALID_ARG, "null x or x_feat");
    if (map == LA_MAP_PERFORMER && !omega)
      return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (map == LA_MAP_PERFORMER)
      e = la::launch_featmap_performer(x, x_feat, omega, rows, d, m, in_dt,
                                       out_dt, s);
    else
      e = la::launch_featmap_elementwise(x, x_feat, rows * d,
                                         map == LA_MAP_ELU1, in_dt, out_dt, s);
    if (e != hipSuccess) return hip_fail(e, "la_featmap launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_featmap");
  }
}

size_t la_forward_workspace_bytes(int B, int H, int64_t n, int d, int d_feat,
                                  la_map map, la_dtype dtype, int causal) {
  try {
    const std::string saved = g_last_error;
    FwdPlan p;
    // The workspace does not depend on decay; size it for the plain variant.
    const la_status st =
        plan_forward(B, H, n, d, d_feat, map, dtype, causal, 0, &p);
    g_last_error = saved;
    if (st != LA_OK) return 0;
    return p.total();
  } catch (...) {
    return 0;
  }
}

size_t la_forward_gated_workspace_bytes(int B, int H, int64_t n, int d,
                                        int d_feat, la_map map,
                                        la_decay_layout layout, la_dtype dtype,
                                        int causal) {
  if (layout == LA_LD_POSITION)
    return la_forward_workspace_bytes(B, H, n, d, d_feat, map, dtype, causal);
  if (layout != LA_LD_CHANNEL && layout != LA_LD_BOTH) return 0;
  try {
    const std::string saved = g_last_error;
    RowPlan p;
    const la_status st = plan_rows(B, H, n, d, d_feat, map, dtype, causal, &p);
    g_last_error = saved;
    if (st != LA_OK) return 0;
    return p.total();
  } catch (...) {
    return 0;
  }
}

la_status la_forward(const void *q, const void *k, const void *v, void *out,
                     int B, int H, int64_t n, int d, int d_feat, la_map map,
                     const float *omega, const float *decay, int causal,
                     la_dtype dtype, void *workspace, void *stream) {
  return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, decay,
                      causal, dtype, workspace, nullptr, nullptr, stream);
}

la_status la_forward_state(const void *q, const void *k, const void *v,
                           void *out, int B, int H, int64_t n, int d,
                           int d_feat, la_map map, const float *omega,
                           const float *decay, int causal, la_dtype dtype,
                           void *workspace, float *mu_out, float *nu_out,
                           void *stream) {
  if (!mu_out || !nu_out)
    return fail(LA_ERR_INVALID_ARG, "la_forward_state needs mu_out and nu_out");
  return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, decay,
                      causal, dtype, workspace, mu_out, nu_out, stream);
}

la_status la_forward_noalloc(const void *q, const void *k, const void *v,
                             void *out, int B, int H, int64_t n, int d,
                             int d_feat, la_map map, const float *omega,
                             const float *decay, int causal, la_dtype dtype,
                             void *stream) {
  try {
    // validate first, so invalid requests touch no device
    FwdPlan p;
    la_status st = plan_forward(B, H, n, d, d_feat, map, dtype, causal,
                                decay != nullptr ? 1 : 0, &p, kScratchBytes);
    if (st != LA_OK) return st;
    if (static_cast<int64_t>(B) * H == 0 || n == 0) return ok();
    if (!q || !k || !v || !out)
      return fail(LA_ERR_INVALID_ARG, "null q, k, v or out");
    if (map == LA_MAP_PERFORMER && !omega)
      return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
    if (p.total() > kScratchBytes)
      return fail(LA_ERR_UNSUPPORTED,
                  "la_forward_noalloc: this call needs a %zu-byte workspace "
                  "(the Performer map with fp32 storage, or sizes the fused "
                  "map is not built for, keep q', k' in it); the static "
                  "scratch holds %zu bytes: use la_forward with a workspace",
                  p.total(), kScratchBytes);
    void *ws = nullptr;
    if (p.total() > 0) {
      st = device_scratch(static_cast<hipStream_t>(stream), &ws);
      if (st != LA_OK) return st;
    }
    return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, decay,
                        causal, dtype, ws, nullptr, nullptr, stream,
                        kScratchBytes);
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_forward_noalloc");
  }
}

la_status la_workspace_check(void *workspace, void *stream) {
  try {
    if (!workspace) return fail(LA_ERR_INVALID_ARG, "null workspace");
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned *word = static_cast<unsigned *>(workspace) + la::kSyncStatusWord;
    unsigned status = 0;
    hipError_t e = hipMemcpyAsync(&status, word, sizeof(status),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "la_workspace_check read");
    if (status == 0) return ok();
    const unsigned zero = 0;
    e = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "la_workspace_check clear");
    return fail(LA_ERR_EXCHANGE, "segment exchange failed since the last "
                "check:%s%s",
                (status & la::kSyncStatusTimeout)
                    ? " a wait for another segment's aggregate gave up "
                      "(those outputs are NaN);" : "",
                (status & la::kSyncStatusCorrupt)
                    ? " the synchronisation area was not zero at the start "
                      "of a call (outputs of that call are unreliable);" : "");
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_workspace_check");
  }
}

void la_set_exchange_spin_limit(unsigned spins) {
  g_spin_limit.store(spins ? spins : la::kDefaultSpinLimit,
                     std::memory_order_relaxed);
}

la_status la_forward_train(const void *q, const void *k, const void *v,
                           void *out, float *den, int B, int H, int64_t n,
                           int d, int d_feat, la_map map, const float *omega,
                           const float *decay, la_dtype dtype, void *workspace,
                           void *stream) {
  if (!den && static_cast<int64_t>(B) * H > 0 && n > 0)
    return fail(LA_ERR_INVALID_ARG, "null den");
  return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, decay, 1,
                      dtype, workspace, nullptr, nullptr, stream, 0, nullptr,
                      den);
}

namespace {
// Workspace of la_backward: G~ rows, then (elu + 1, column-block kernel)
// K' and Q', then the segment aggregates of the segmented roles (and, for
// a decay per position, each segment's sum of log2 gamma).
size_t backward_ws(int64_t units, int64_t n, int d, int map, int dtype,
                   size_t *kf_off, size_t *agg_off = nullptr) {
  const size_t es = elem_size(dtype);
  const size_t g = align256(static_cast<size_t>(units * n) *
                            la::backward_gwidth(d) * es);
  const size_t f = align256(static_cast<size_t>(units * n) * d * es);
  const int nseg = la::backward_segments(units, n, d, dtype);
  // the segmented roles map k, q themselves: no K', Q' rows
  const size_t feats = map == LA_MAP_ELU1 && nseg == 0 ? 2 * f : 0;
  const size_t agg =
      align256(la::backward_agg_floats(units, nseg) * sizeof(float));
  if (kf_off) *kf_off = g;
  if (agg_off) *agg_off = g + feats;
  return g + feats + agg;
}
// Workspace of la_backward with the Performer map: G~ rows, then K', Q'
// (dtype) and the feature gradients dq', dk' (fp32), d_feat values per row
// each; *fbytes and *gbytes are the sizes of one feature and one feature
// gradient buffer.
size_t backward_ws_performer(int64_t units, int64_t n, int d, int d_feat,
                             int dtype, size_t *fbytes, size_t *gbytes) {
  const size_t es = elem_size(dtype);
  const size_t g = align256(static_cast<size_t>(units * n) *
                            la::backward_gwidth(d) * es);
  const size_t f = align256(static_cast<size_t>(units * n) * d_feat * es);
  const size_t fg = align256(static_cast<size_t>(units * n) * d_feat * 4);
  if (fbytes) *fbytes = f;
  if (gbytes) *gbytes = fg;
  return g + 2 * f + 2 * fg;
}
}  // namespace

size_t la_backward_workspace_bytes(int B, int H, int64_t n, int d, int d_feat,
                                   la_map map, la_dtype dtype) {
  if (B <= 0 || H <= 0 || n <= 0 || !valid_dtype(dtype) || !valid_map(map))
    return 0;
  if (map == LA_MAP_PERFORMER ? !la::backward_performer_supported(d, d_feat)
                              : !la::backward_supported(d, d_feat))
    return 0;
  const int64_t units = static_cast<int64_t>(B) * H;
  if (units * n > (int64_t{1} << 46) || units > (int64_t{1} << 26)) return 0;
  if (map == LA_MAP_PERFORMER)
    return backward_ws_performer(units, n, d, d_feat, dtype, nullptr, nullptr);
  return backward_ws(units, n, d, map, dtype, nullptr);
}

// la_backward with the Performer map: K' = phi(k), Q' = phi(q) into the
// workspace, the three roles over them (dq', dk' to the workspace, dv to
// its output), then dq, dk through the map.
static la_status backward_performer(const void *q, const void *k,
                                    const void *v, const void *out,
                                    const float *den, const void *dout,
                                    void *dq, void *dk, void *dv, int B, int H,
                                    int64_t n, int d, int d_feat,
                                    const float *omega, const float *decay,
                                    const float *lam, la_dtype dtype,
                                    void *workspace, void *stream) {
  if (!la::backward_performer_supported(d, d_feat))
    return fail(LA_ERR_UNSUPPORTED,
                "la_backward PERFORMER: d in {32, 64, 128}, d_feat in {32, "
                "64, 128, 256}, d * d_feat <= 16384 are built (got d=%d "
                "d_feat=%d)", d, d_feat);
  const int64_t units = static_cast<int64_t>(B) * H;
  if (units == 0 || n == 0) return ok();
  if (units * n > (int64_t{1} << 46) || units > (int64_t{1} << 26))
    return fail(LA_ERR_UNSUPPORTED, "sizes too large");
  if (!q || !k || !v || !out || !den || !dout || !dq || !dk || !dv)
    return fail(LA_ERR_INVALID_ARG, "null pointer argument");
  if (!omega) return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
  size_t fb = 0, gb = 0;
  const size_t total =
      backward_ws_performer(units, n, d, d_feat, dtype, &fb, &gb);
  if (!workspace)
    return fail(LA_ERR_WORKSPACE, "la_backward: workspace of %zu bytes required",
                total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  const size_t g = total - 2 * fb - 2 * gb;
  la::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.den = den;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.decay = lam ? nullptr : decay;
  a.lam = lam;
  a.H = H;
  a.n = n;
  a.dqk = d;
  a.elu1 = 0;
  a.gt = ws;
  a.kf = ws + g;
  a.qf = ws + g + fb;
  a.dqf = ws + g + 2 * fb;
  a.dkf = ws + g + 2 * fb + gb;
  a.omega = omega;
  a.nseg = 0;
  a.agg = nullptr;
  hipError_t e = la::launch_featmap_performer(k, a.kf, omega, units * n, d,
                                              d_feat, dtype, dtype, s);
  if (e == hipSuccess)
    e = la::launch_featmap_performer(q, a.qf, omega, units * n, d, d_feat,
                                     dtype, dtype, s);
  if (e != hipSuccess) return hip_fail(e, "la_backward feature map");
  e = la::launch_backward_performer(a, units, d, d_feat, dtype == LA_BF16 ? 1 : 0, s);
  if (e != hipSuccess) return hip_fail(e, "la_backward launch");
  return ok();
}

size_t la_backward_gated_workspace_bytes(int B, int H, int64_t n, int d,
                                         int d_feat, la_map map,
                                         la_dtype dtype) {
  if (B <= 0 || H <= 0 || n <= 0 || !valid_dtype(dtype) || !valid_map(map))
    return 0;
  if (map == LA_MAP_PERFORMER ? !la::backward_performer_supported(d, d_feat)
                              : !la::backward_supported(d, d_feat))
    return 0;
  const int64_t units = static_cast<int64_t>(B) * H;
  if (units * n > (int64_t{1} << 46) || units > (int64_t{1} << 26)) return 0;
  if (map == LA_MAP_PERFORMER)
    return backward_ws_performer(units, n, d, d_feat, dtype, nullptr, nullptr);
  return backward_ws(units, n, d, map, dtype, nullptr);
}

// la_backward (decay [H] or null, lam null) and la_backward_gated (lam, a
// decay per position, [B][H][n]).
static la_status backward_impl(const void *q, const void *k, const void *v,
                               const void *out, const float *den,
                               const void *dout, void *dq, void *dk, void *dv,
                               int B, int H, int64_t n, int d, int d_feat,
                               la_map map, const float *omega,
                               const float *decay, const float *lam,
                               la_dtype dtype, void *workspace, void *stream) {
  try {
    if (B < 0 || H < 0 || n < 0)
      return fail(LA_ERR_INVALID_ARG, "negative size");
    if (!valid_map(map)) return fail(LA_ERR_INVALID_ARG, "unknown map %d", map);
    if (!valid_dtype(dtype))
      return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (d <= 0 || d_feat <= 0)
      return fail(LA_ERR_INVALID_ARG, "non-positive d=%d d_feat=%d", d, d_feat);
    if (map == LA_MAP_ELU1 && d_feat != d)
      return fail(LA_ERR_INVALID_ARG, "ELU1 needs d_feat == d");
    if (map == LA_MAP_PERFORMER)
      return backward_performer(q, k, v, out, den, dout, dq, dk, dv, B, H, n,
                                d, d_feat, omega, decay, lam, dtype,
                                workspace, stream);
    if (!la::backward_supported(d, d_feat))
      return fail(LA_ERR_UNSUPPORTED,
                  "la_backward: d = d_feat in {16, 32, 64, 128} is built "
                  "(got d=%d d_feat=%d)", d, d_feat);
    const int64_t units = static_cast<int64_t>(B) * H;
    if (units == 0 || n == 0) return ok();
    if (units * n > (int64_t{1} << 46) || units > (int64_t{1} << 26))
      return fail(LA_ERR_UNSUPPORTED, "sizes too large");
    if (!q || !k || !v || !out || !den || !dout || !dq || !dk || !dv)
      return fail(LA_ERR_INVALID_ARG, "null pointer argument");
    const bool gated = lam != nullptr;
    if (!workspace)
      return fail(LA_ERR_WORKSPACE, "la_backward: workspace of %zu bytes required",
                  backward_ws(units, n, d, map, dtype, nullptr));
    size_t kf_off = 0, agg_off = 0;
    const size_t fbytes = align256(static_cast<size_t>(units * n) * d *
                                   elem_size(dtype));
    backward_ws(units, n, d, map, dtype, &kf_off, &agg_off);
    la::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.den = den;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.decay = gated ? nullptr : decay;
    a.lam = lam;
    a.H = H;
    a.n = n;
    a.dqk = d;
    a.elu1 = map == LA_MAP_ELU1;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    a.gt = ws;
    a.nseg = la::backward_segments(units, n, d, dtype);
    // K', Q' rows only where the column-block kernel reads them
    const bool feats = a.elu1 && a.nseg == 0;
    a.kf = feats ? ws + kf_off : const_cast<void *>(k);
    a.qf = feats ? ws + kf_off + fbytes : const_cast<void *>(q);
    a.agg = reinterpret_cast<float *>(ws + agg_off);
    const hipError_t e = la::launch_backward(a, units, d, dtype,
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "la_backward launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_backward");
  }
}

la_status la_backward(const void *q, const void *k, const void *v,
                      const void *out, const float *den, const void *dout,
                      void *dq, void *dk, void *dv, int B, int H, int64_t n,
                      int d, int d_feat, la_map map, const float *omega,
                      const float *decay, la_dtype dtype, void *workspace,
                      void *stream) {
  return backward_impl(q, k, v, out, den, dout, dq, dk, dv, B, H, n, d,
                       d_feat, map, omega, decay, nullptr, dtype, workspace,
                       stream);
}

la_status la_backward_gated(const void *q, const void *k, const void *v,
                            const void *out, const float *den,
                            const void *dout, void *dq, void *dk, void *dv,
                            int B, int H, int64_t n, int d, int d_feat,
                            la_map map, const float *omega,
                            const float *log_decay, la_decay_layout layout,
                            la_dtype dtype, void *workspace, void *stream) {
  if (layout != LA_LD_CHANNEL && layout != LA_LD_POSITION &&
      layout != LA_LD_BOTH)
    return fail(LA_ERR_INVALID_ARG, "unknown decay layout %d", layout);
  if (layout != LA_LD_POSITION)
    return fail(LA_ERR_UNSUPPORTED,
                "la_backward_gated: only LA_LD_POSITION is built");
  if (!log_decay && static_cast<int64_t>(B) * H > 0 && n > 0)
    return fail(LA_ERR_INVALID_ARG, "null log_decay");
  return backward_impl(q, k, v, out, den, dout, dq, dk, dv, B, H, n, d,
                       d_feat, map, omega, nullptr, log_decay, dtype,
                       workspace, stream);
}

la_status la_forward_gated_train(const void *q, const void *k, const void *v,
                                 void *out, float *den, int B, int H,
                                 int64_t n, int d, int d_feat, la_map map,
                                 const float *omega, const float *log_decay,
                                 la_decay_layout layout, la_dtype dtype,
                                 void *workspace, void *stream) {
  if (layout != LA_LD_CHANNEL && layout != LA_LD_POSITION &&
      layout != LA_LD_BOTH)
    return fail(LA_ERR_INVALID_ARG, "unknown decay layout %d", layout);
  if (layout != LA_LD_POSITION)
    return fail(LA_ERR_UNSUPPORTED,
                "la_forward_gated_train: only LA_LD_POSITION is built");
  const bool empty = static_cast<int64_t>(B) * H <= 0 || n <= 0;
  if (!den && !empty) return fail(LA_ERR_INVALID_ARG, "null den");
  if (!log_decay && !empty) return fail(LA_ERR_INVALID_ARG, "null log_decay");
  return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, nullptr, 1,
                      dtype, workspace, nullptr, nullptr, stream, 0, log_decay,
                      den);
}

la_status la_forward_gated(const void *q, const void *k, const void *v,
                           void *out, int B, int H, int64_t n, int d,
                           int d_feat, la_map map, const float *omega,
                           const float *log_decay, la_decay_layout layout,
                           int causal, la_dtype dtype, void *workspace,
                           float *mu_out, float *nu_out, void *stream) {
  if (layout != LA_LD_CHANNEL && layout != LA_LD_POSITION &&
      layout != LA_LD_BOTH)
    return fail(LA_ERR_INVALID_ARG, "unknown decay layout %d", layout);
  if ((mu_out == nullptr) != (nu_out == nullptr))
    return fail(LA_ERR_INVALID_ARG, "mu_out and nu_out go together");
  if (!log_decay && static_cast<int64_t>(B) * H > 0 && n > 0)
    return fail(LA_ERR_INVALID_ARG, "null log_decay");
  if (layout != LA_LD_POSITION)
    return forward_rows_impl(q, k, v, out, B, H, n, d, d_feat, map, omega,
                             log_decay, layout == LA_LD_BOTH ? 1 : 0, causal,
                             dtype, workspace, mu_out, nu_out, stream);
  return forward_impl(q, k, v, out, B, H, n, d, d_feat, map, omega, nullptr,
                      causal, dtype, workspace, mu_out, nu_out, stream, 0,
                      log_decay ? log_decay : nullptr);
}

// la_decode_step and la_decode_step_gated: ld_layout < 0 for the former
// (decay [H] or NULL), else the layout of log_decay.
static la_status decode_impl(float *mu, float *nu, const void *q, const void *k,
                             const void *v, void *out, int S, int H, int d,
                             int d_feat, int map, const float *omega,
                             const float *decay, int dtype, void *stream,
                             int ld_layout) {
  try {
    if (S < 0 || H < 0) return fail(LA_ERR_INVALID_ARG, "negative size");
    if (!valid_map(map)) return fail(LA_ERR_INVALID_ARG, "unknown map %d", map);
    if (!valid_dtype(dtype)) return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (d <= 0 || d_feat <= 0)
      return fail(LA_ERR_INVALID_ARG, "non-positive d=%d d_feat=%d", d, d_feat);
    if (map == LA_MAP_ELU1 && d_feat != d)
      return fail(LA_ERR_INVALID_ARG, "ELU1 needs d_feat == d");
    if (!supported_d(d) || !la::decode_supported(d, d_feat))
      return fail(LA_ERR_UNSUPPORTED, "unsupported d=%d d_feat=%d", d, d_feat);
    const int64_t units = static_cast<int64_t>(S) * H;
    if (units == 0) return ok();
    if (units > (int64_t{1} << 31) - 1)
      return fail(LA_ERR_UNSUPPORTED, "too many units");
    if (!mu || !nu || !q || !k || !v || !out)
      return fail(LA_ERR_INVALID_ARG, "null pointer argument");
    if (map == LA_MAP_PERFORMER && !omega)
      return fail(LA_ERR_INVALID_ARG, "PERFORMER needs omega");
    if (ld_layout >= 0 && !decay)
      return fail(LA_ERR_INVALID_ARG, "null log_decay");
    const hipError_t e = la::launch_decode(
        mu, nu, q, k, v, out, units, H, d, d_feat, map, omega, decay, dtype,
        static_cast<hipStream_t>(stream), ld_layout);
    if (e != hipSuccess) return hip_fail(e, "la_decode_step launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in la_decode_step");
  }
}

la_status la_decode_step(float *mu, float *nu, const void *q, const void *k,
                         const void *v, void *out, int S, int H, int d,
                         int d_feat, la_map map, const float *omega,
                         const float *decay, la_dtype dtype, void *stream) {
  return decode_impl(mu, nu, q, k, v, out, S, H, d, d_feat, map, omega, decay,
                     dtype, stream, -1);
}

la_status la_decode_step_gated(float *mu, float *nu, const void *q,
                               const void *k, const void *v, void *out, int S,
                               int H, int d, int d_feat, la_map map,
                               const float *omega, const float *log_decay,
                               la_decay_layout layout, la_dtype dtype,
                               void *stream) {
  if (layout != LA_LD_CHANNEL && layout != LA_LD_POSITION &&
      layout != LA_LD_BOTH)
    return fail(LA_ERR_INVALID_ARG, "unknown decay layout %d", layout);
  return decode_impl(mu, nu, q, k, v, out, S, H, d, d_feat, map, omega,
                     log_decay, dtype, stream, static_cast<int>(layout));
}

}  // extern "C"
