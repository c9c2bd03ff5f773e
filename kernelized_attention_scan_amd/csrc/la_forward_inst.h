// Launchers and the (d, d_feat) instance table of the fused forward, for one
// storage type (included once per type by la_forward_*.hip).
#pragma once

#include "la_forward.h"
#include "la_internal.h"

namespace la {

// One (storage type, d, d_feat, decay, map) instance; MAP is the feature map
// applied to q and k while staging them (kMapFeatures: none).
template <typename T, int D, int DF, bool DECAY, int MAP>
struct FwdVariant {
  using F = FwdShape<T, D, DF, DECAY, MAP>;

  static const void *kernel(bool causal, bool multi) {
    if (causal)
      return multi
          ? reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, true, true, DECAY, MAP>)
          : reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, true, false, DECAY, MAP>);
    return reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, false, true, DECAY, MAP>);
  }

  // Resident-key instance (causal, several segments of at most KRES chunks).
  static const void *kernel_res() {
    if constexpr (F::KRES > 0)
      return reinterpret_cast<const void *>(
          &la_fwd_kernel<T, D, DF, true, true, DECAY, MAP, true>);
    return kernel(true, true);
  }

  // Raise the dynamic-LDS limit of every instance once (above 64 KiB).
  static hipError_t set_lds() {
    static const hipError_t once = [] {
      for (const void *k : {kernel(true, true), kernel(true, false),
                            kernel(false, true), kernel_res()}) {
        const hipError_t e = hipFuncSetAttribute(
            k, hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(F::lds_bytes));
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }();
    return once;
  }

  // Workgroups of the non-causal multi-segment kernel resident at once.
  static hipError_t capacity(int64_t *cap) {
    static int per_cu = -1;
    static int cus = 0;
    if (per_cu < 0) {
      int dev = 0, n = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, kernel(false, true), kThreads, F::lds_bytes);
      if (e != hipSuccess) return e;
      per_cu = n;
    }
    *cap = static_cast<int64_t>(per_cu) * cus;
    return hipSuccess;
  }

  static hipError_t run(const FwdArgs &args, int64_t units, int causal,
                        hipStream_t s) {
    hipError_t e = set_lds();
    if (e != hipSuccess) return e;
    FwdArgs a = args;
    if (a.nseg > 1 && !causal) {
      // The non-causal exchange waits on every segment, so every workgroup
      // must be resident: shrink the split to what fits (the workspace was
      // sized for the largest split) and launch cooperatively.
      int64_t cap = 0;
      e = capacity(&cap);
      if (e != hipSuccess) return e;
      if (units * a.nseg > cap) {
        int64_t nseg = cap / units;
        if (nseg < 1) nseg = 1;
        const int64_t nch = (a.n + F::C - 1) / F::C;
        const int64_t cps = (nch + nseg - 1) / nseg;
        a.seg_len = cps * F::C;
        a.nseg = static_cast<int>((a.n + a.seg_len - 1) / a.seg_len);
      }
    }
    const dim3 grid(static_cast<unsigned>(units * a.nseg)), block(kThreads);
    if (causal) {
      // One segment: no exchange.  Several: segments are numbered in start
      // order, so a plain launch cannot deadlock.
      if (a.nseg == 1) {
        hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, true, false, DECAY, MAP>),
                           grid, block, F::lds_bytes, s, a);
        return hipGetLastError();
      }
      if constexpr (F::KRES > 0) {
        if (a.seg_len <= static_cast<int64_t>(F::KRES) * F::C) {
          hipLaunchKernelGGL(
              (la_fwd_kernel<T, D, DF, true, true, DECAY, MAP, true>), grid,
              block, F::lds_bytes, s, a);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, true, true, DECAY, MAP>),
                         grid, block, F::lds_bytes, s, a);
      return hipGetLastError();
    }
    if (a.nseg == 1) {  // non-causal, one segment: no exchange executes
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, false, true, DECAY, MAP>),
                         grid, block, F::lds_bytes, s, a);
      return hipGetLastError();
    }
    void *params[] = {&a};
    return hipLaunchCooperativeKernel(kernel(false, true), grid, block, params,
                                      F::lds_bytes, s);
  }
};

// Launch set of one (storage type, d, d_feat): PERF selects the instances
// with the Performer map fused, else the ones for features or elu + 1.
template <typename T, int D, int DF, bool PERF = false>
struct FwdRunner {
  static constexpr int MAP0 = PERF ? kMapPerformer : kMapFeatures;
  using P = FwdShape<T, D, DF, false, MAP0>;
  using Q = FwdShape<T, D, DF, true, MAP0>;

  template <int MAP>
  static hipError_t run_map(const FwdArgs &a, int64_t units, int causal,
                            hipStream_t s) {
    if (a.decay) {
      if constexpr (Q::fits)
        return FwdVariant<T, D, DF, true, MAP>::run(a, units, causal, s);
      else
        return hipErrorInvalidValue;
    }
    return FwdVariant<T, D, DF, false, MAP>::run(a, units, causal, s);
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
      // chunks of the decayed variant too
      static_assert(!Q::fits || P::C % Q::C == 0, "chunk lengths compatible");
      static const FwdOps o = {P::C, P::SLOT, Q::fits, &run};
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
