// Launchers and the (d, d_feat) instance table of the forward with a decay
// per state row, for one storage type (included once per type).
#pragma once

#include "la_forward_rows.h"

namespace la {

__global__ __launch_bounds__(256) void la_fwd_rows_carry_kernel(
    float *agg, int nseg, int nsum, int slot, int nstate, int dfp, int nft,
    int d, int df, float *mu_out, float *nu_out);

template <typename T, int D, int DF>
struct RowRunner {
  using S = RowShape<T, D, DF>;

  template <int PHASE, bool PP>
  static const void *kernel() {
    return reinterpret_cast<const void *>(&la_fwd_rows_kernel<T, D, DF, PHASE, PP>);
  }

  // Raise the dynamic-LDS limit of every instance once where it exceeds the
  // default (a function-local static: C++'s thread-safe initialisation).
  static hipError_t set_lds() {
    static const hipError_t once = [] {
      if (S::lds_bytes <= 64 * 1024) return hipSuccess;
      for (const void *k : {kernel<0, false>(), kernel<0, true>(),
                            kernel<1, false>(), kernel<1, true>(),
                            kernel<2, false>()}) {
        const hipError_t e = hipFuncSetAttribute(
            k, hipFuncAttributeMaxDynamicSharedMemorySize, S::lds_bytes);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }();
    return once;
  }

  template <int PHASE>
  static void launch(const RowArgs &a, dim3 grid, hipStream_t s) {
    if (a.per_position)
      hipLaunchKernelGGL((la_fwd_rows_kernel<T, D, DF, PHASE, true>), grid,
                         dim3(kRowThreads), S::lds_bytes, s, a);
    else
      hipLaunchKernelGGL((la_fwd_rows_kernel<T, D, DF, PHASE, false>), grid,
                         dim3(kRowThreads), S::lds_bytes, s, a);
  }

  static hipError_t run(const RowArgs &a, int64_t units, int causal,
                        hipStream_t s) {
    hipError_t e = set_lds();
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(units * a.nseg));
    if (!causal || a.nseg > 1) {
      // every segment's aggregate (causal: the last one has no reader), then
      // the incoming state of every segment and the total
      RowArgs b = a;
      b.skip_last = causal ? 1 : 0;
      launch<1>(b, grid, s);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const dim3 cgrid(static_cast<unsigned>(
          units * ((S::NSTATE + S::DFP + 255) / 256)));
      hipLaunchKernelGGL(la_fwd_rows_carry_kernel, cgrid, dim3(256), 0, s,
                         a.agg, a.nseg, causal ? a.nseg - 1 : a.nseg, S::SLOT,
                         S::NSTATE, S::DFP, S::NFT, D, DF,
                         causal ? nullptr : a.mu_out,
                         causal ? nullptr : a.nu_out);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (causal) {
      launch<0>(a, grid, s);
    } else {
      hipLaunchKernelGGL((la_fwd_rows_kernel<T, D, DF, 2, false>), grid,
                         dim3(kRowThreads), S::lds_bytes, s, a);
    }
    return hipGetLastError();
  }

  static const RowOps *ops() {
    static const RowOps o = {S::SLOT, &run};
    return &o;
  }
};

template <typename T, int D>
const RowOps *row_ops_by_feat(int d_feat) {
  switch (d_feat) {
    case 16: return RowRunner<T, D, 16>::ops();
    case 32: return RowRunner<T, D, 32>::ops();
    case 64: return RowRunner<T, D, 64>::ops();
    case 128: return RowRunner<T, D, 128>::ops();
    case 256: return RowRunner<T, D, 256>::ops();
    default: return nullptr;
  }
}

}  // namespace la
