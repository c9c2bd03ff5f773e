// Launchers and the (d, d_feat) instance table of the chunked forward, for
// one storage type LA_T (included once per type by la_forward_*.hip).
#pragma once

#include "la_forward.h"
#include "la_internal.h"

namespace la {

template <typename T, int D, int DF>
struct FwdRunner {
  using F = FwdShape<T, D, DF>;

  static hipError_t set_lds() {
    // Raise the dynamic-LDS limit once per kernel instance (above 64 KiB).
    static const hipError_t once = [] {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, true>),
          hipFuncAttributeMaxDynamicSharedMemorySize,
          static_cast<int>(F::lds_fwd));
      if (e == hipSuccess)
        e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&la_fwd_kernel<T, D, DF, false>),
            hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(F::lds_fwd));
      if (e == hipSuccess)
        e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&la_agg_kernel<T, D, DF>),
            hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(F::lds_agg));
      return e;
    }();
    return once;
  }

  static hipError_t run(const FwdArgs &a, int64_t units, int causal,
                        hipStream_t s) {
    hipError_t e = set_lds();
    if (e != hipSuccess) return e;
    const int64_t nblk = units * a.nseg;
    if (a.states) {
      hipLaunchKernelGGL((la_agg_kernel<T, D, DF>), dim3(nblk), dim3(kThreads),
                         F::lds_agg, s, a);
      const hipError_t es = launch_scan(a.states, a.decay, a.H, a.n, a.seg_len,
                                        a.nseg, units, F::SLOT, F::SLOT_USED,
                                        s);
      if (es != hipSuccess) return es;
    }
    if (causal)
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, true>), dim3(nblk),
                         dim3(kThreads), F::lds_fwd, s, a);
    else
      hipLaunchKernelGGL((la_fwd_kernel<T, D, DF, false>), dim3(nblk),
                         dim3(kThreads), F::lds_fwd, s, a);
    return hipGetLastError();
  }

  static const FwdOps *ops() {
    if constexpr (!F::fits) {
      return nullptr;
    } else {
      static const FwdOps o = {F::C, F::SLOT, F::lds_fwd, F::lds_agg, &run};
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
