// bf16-storage instances of the chunked forward (bf16 matrix-core operands,
// fp32 accumulation and state).
#include "la_forward_inst.h"

namespace la {
const FwdOps *fwd_ops_bf16(int d, int d_feat) {
  return fwd_ops_for<bf16>(d, d_feat);
}
}  // namespace la
