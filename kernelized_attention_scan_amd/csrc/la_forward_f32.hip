// fp32-storage instances of the chunked forward (fp32 matrix-core operands).
#include "la_forward_inst.h"

namespace la {
const FwdOps *fwd_ops_f32(int d, int d_feat) {
  return fwd_ops_for<float>(d, d_feat);
}
}  // namespace la
