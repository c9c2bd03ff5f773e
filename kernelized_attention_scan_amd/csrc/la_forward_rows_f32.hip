// fp32-storage instances of the forward with a decay per state row.
#include "la_forward_rows_inst.h"

namespace la {
const RowOps *row_ops_f32(int d, int d_feat) {
  switch (d) {
    case 16: return row_ops_by_feat<float, 16>(d_feat);
    case 32: return row_ops_by_feat<float, 32>(d_feat);
    case 64: return row_ops_by_feat<float, 64>(d_feat);
    case 128: return row_ops_by_feat<float, 128>(d_feat);
    default: return nullptr;
  }
}
}  // namespace la
