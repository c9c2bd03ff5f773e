// Launchers and the (d, d_feat) instance table of the fused forward, for one
// storage type (included once per type by la_forward_*.hip).
#pragma once

#include "la_forward.h"
#include "la_internal.h"

namespace la {

// One (storage type, d, d_feat, decay mode, map) instance; DK is the decay
// mode of FwdShape, MAP the feature map applied to q and k while staging
// them (kMapFeatures: none).  VS > 1: the value columns are split into VS
// parts of D columns, each its own set of workgroups.
template <typename T, int D, int DF, int DK, int MAP, int VS = 1>
struct FwdVariant {
  using F = FwdShape<T, D, DF, DK, MAP>;

  static const void *kernel(bool causal, bool multi) {
    if (causal)
      return multi
          ? reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, true, true, DK, MAP, false, 0, VS>)
          : reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, true, false, DK, MAP, false, 0, VS>);
    return reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 0, VS>);
  }

  // Non-causal segmented forward as two launches: the aggregates, then the
  // readout against their total.
  static const void *kernel_split(int split) {
    return split == 1
        ? reinterpret_cast<const void *>(
              &la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 1, VS>)
        : reinterpret_cast<const void *>(
              &la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 2, VS>);
  }

  // Resident-key instance (causal, several segments of at most KRES chunks).
  static const void *kernel_res() {
    if constexpr (F::KRES > 0)
      return reinterpret_cast<const void *>(
          &la_fwd_kernel<T, D, DF, true, true, DK, MAP, true, 0, VS>);
    return kernel(true, true);
  }

  // Raise the dynamic-LDS limit of every instance once (above 64 KiB); a
  // function-local static, so the first call does it under C++'s
  // thread-safe initialisation.
  static hipError_t set_lds() {
    static const hipError_t once = [] {
      for (const void *k : {kernel(true, true), kernel(true, false),
                            kernel(false, true), kernel_res(),
                            kernel_split(1), kernel_split(2)}) {
        const hipError_t e = hipFuncSetAttribute(
            k, hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(F::lds_bytes));
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }();
    return once;
  }

  static hipError_t run(const FwdArgs &a, int64_t units, int causal,
                        hipStream_t s) {
    hipError_t e = set_lds();
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(units * VS * a.nseg)),
        block(kThreads);
    if (causal) {
      // One segment: no exchange.  Several: segments are numbered in start
      // order, so a plain launch cannot deadlock.
      if (a.nseg == 1) {
        hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, true, false, DK, MAP, false, 0, VS>),
                           grid, block, F::lds_bytes, s, a);
        return hipGetLastError();
      }
      if constexpr (F::KRES > 0) {
        if (a.seg_len <= static_cast<int64_t>(F::KRES) * F::C) {
          hipLaunchKernelGGL(
              (la_fwd_kernel<T, D, DF, true, true, DK, MAP, true, 0, VS>), grid,
              block, F::lds_bytes, s, a);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, true, true, DK, MAP, false, 0, VS>),
                         grid, block, F::lds_bytes, s, a);
      return hipGetLastError();
    }
    if (a.nseg == 1) {  // non-causal, one segment: no exchange executes
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 0, VS>),
                         grid, block, F::lds_bytes, s, a);
      return hipGetLastError();
    }
    // Non-causal, several segments: every readout needs every segment's
    // aggregate, so the aggregates come from a launch of their own and the
    // readout launch after it on the same stream reads them; no workgroup
    // ever waits for another.
    hipLaunchKernelGGL(
        (la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 1, VS>), grid,
        block, F::lds_bytes, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(
        (la_fwd_kernel<T, D, DF, false, true, DK, MAP, false, 2, VS>), grid,
        block, F::lds_bytes, s, a);
    return hipGetLastError();
  }
};

// Launch set of one (storage type, d, d_feat): PERF selects the instances
// with the Performer map fused, else the ones for features or elu + 1.
// Where no instance of the full value width fits LDS (fp32 storage, d = 128,
// d' = 256: the fp32 S^T copy alone is 147 KiB) the value columns are split
// in two halves (VS = 2), each its own computation over all of q', k'.
template <typename T, int D, int DF, bool PERF = false>
struct FwdRunner {
  static constexpr int MAP0 = PERF ? kMapPerformer : kMapFeatures;
  static constexpr int VS =
      !PERF && !FwdShape<T, D, DF, 0, MAP0>::fits && D >= 32 ? 2 : 1;
  static constexpr int DP = D / VS;       // value columns per part
  using P = FwdShape<T, DP, DF, 0, MAP0>;  // no decay
  using Q = FwdShape<T, DP, DF, 1, MAP0>;  // one decay per head
  using R = FwdShape<T, DP, DF, 2, MAP0>;  // a decay per position

  template <int MAP>
  static hipError_t run_map(const FwdArgs &a, int64_t units, int causal,
                            hipStream_t s) {
    if (a.log_decay) {
      if constexpr (R::fits)
        return FwdVariant<T, DP, DF, 2, MAP, VS>::run(a, units, causal, s);
      else
        return hipErrorInvalidValue;
    }
    if (a.decay) {
      if constexpr (Q::fits)
        return FwdVariant<T, DP, DF, 1, MAP, VS>::run(a, units, causal, s);
      else
        return hipErrorInvalidValue;
    }
    return FwdVariant<T, DP, DF, 0, MAP, VS>::run(a, units, causal, s);
  }

  // elu + 1 instances exist only for d_feat == d (the map keeps the width).
  static hipError_t run(const FwdArgs &a, int64_t units, int causal,
                        hipStream_t s) {
    if constexpr (PERF) {
      return run_map<kMapPerformer>(a, units, causal, s);
    } else {
      if (a.elu1) {
        if constexpr (D == DF)
          return run_map<kMapElu>(a, units, causal, s);
        else
          return hipErrorInvalidValue;
      }
      return run_map<kMapFeatures>(a, units, causal, s);
    }
  }

  static const FwdOps *ops() {
    if constexpr (!P::fits) {
      return nullptr;
    } else {
      // the split is planned with P's chunk length; segments must hold whole
      // chunks of the decayed variants too
      static_assert(!Q::fits || P::C % Q::C == 0, "chunk lengths compatible");
      static_assert(!R::fits || P::C % R::C == 0, "chunk lengths compatible");
      static const FwdOps o = {P::C, P::SLOT, Q::fits, R::fits, VS, &run};
      return &o;
    }
  }
};

template <typename T, int D>
const FwdOps *fwd_ops_by_feat(int d_feat) {
  switch (d_feat) {
    case 16: return FwdRunner<T, D, 16>::ops();
    case 32: return FwdRunner<T, D, 32>::ops();
    case 64: return FwdRunner<T, D, 64>::ops();
    case 128: return FwdRunner<T, D, 128>::ops();
    case 256: return FwdRunner<T, D, 256>::ops();
    default: return nullptr;
  }
}

template <typename T>
const FwdOps *fwd_ops_for(int d, int d_feat) {
  switch (d) {
    case 16: return fwd_ops_by_feat<T, 16>(d_feat);
    case 32: return fwd_ops_by_feat<T, 32>(d_feat);
    case 64: return fwd_ops_by_feat<T, 64>(d_feat);
    case 128: return fwd_ops_by_feat<T, 128>(d_feat);
    default: return nullptr;
  }
}

}  // namespace la
