// bf16-storage instances of the chunked forward with the Performer feature
// map fused into it: q and k of width d are mapped to d_feat random features
// on chip, so the features never go through memory.
#include "la_forward_inst.h"

namespace la {
namespace {
template <int D>
const FwdOps *pf_by_feat(int d_feat) {
  switch (d_feat) {
    case 32: return FwdRunner<bf16, D, 32, true>::ops();
    case 64: return FwdRunner<bf16, D, 64, true>::ops();
    case 128: return FwdRunner<bf16, D, 128, true>::ops();
    case 256: return FwdRunner<bf16, D, 256, true>::ops();
    default: return nullptr;
  }
}
}  // namespace

const FwdOps *fwd_ops_bf16_performer(int d, int d_feat) {
  switch (d) {
    case 32: return pf_by_feat<32>(d_feat);
    case 64: return pf_by_feat<64>(d_feat);
    case 128: return pf_by_feat<128>(d_feat);
    default: return nullptr;
  }
}
}  // namespace la
