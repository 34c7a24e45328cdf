// rope_kernels_f32_row.hip -- the row, scalar and table kernels for float32 storage
// (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_ROW_ENTRY_POINTS(, float)
}  // namespace rope
