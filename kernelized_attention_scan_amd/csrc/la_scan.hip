// Exclusive prefix over the segments of each (batch, head) unit.
//
// Segment s of a unit has aggregate A_s, the state its positions produce from a
// zero state (eqs 7-8 or 10-11 of "2.2 Linear Attention", efficient2 page,
// applied over the segment).  The state entering segment s is
//   I_0 = 0,   I_{s+1} = g^{len_s} I_s + A_s,
// the same recurrence one level up.  Each thread owns one fp32 element of the
// state slot (tiles of mu, then nu) of one unit and walks the segments in
// order; slot nseg receives the total, the state after the last position.
#include "la_device.h"
#include "la_internal.h"

namespace la {

namespace {
constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kScanThreads) void la_scan_kernel(
    float *states, const float *decay, int H, int64_t n, int64_t seg_len,
    int nseg, int slot, int used) {
  const int eblk = (used + kScanThreads - 1) / kScanThreads;
  const int64_t unit = blockIdx.x / eblk;
  const int e = (blockIdx.x % eblk) * kScanThreads + threadIdx.x;
  if (e >= used) return;
  const int h = static_cast<int>(unit % H);
  const float g = decay ? decay[h] : 1.f;
  const float lg = log2f(g);
  float *p = states + unit * (nseg + 1) * static_cast<int64_t>(slot) + e;
  float run = 0.f;
  for (int s = 0; s < nseg; ++s) {
    const int64_t len = min(seg_len, n - s * seg_len);
    const float x = p[static_cast<int64_t>(s) * slot];
    p[static_cast<int64_t>(s) * slot] = run;
    run = pow_int(g, lg, len) * run + x;
  }
  p[static_cast<int64_t>(nseg) * slot] = run;
}
}  // namespace

hipError_t launch_scan(float *states, const float *decay, int H, int64_t n,
                       int64_t seg_len, int nseg, int64_t units, int slot,
                       int used, hipStream_t s) {
  const int64_t eblk = (used + kScanThreads - 1) / kScanThreads;
  hipLaunchKernelGGL(la_scan_kernel, dim3(eblk * units), dim3(kScanThreads), 0,
                     s, states, decay, H, n, seg_len, nseg, slot, used);
  return hipGetLastError();
}

}  // namespace la
