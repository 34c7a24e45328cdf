// rope_kernels_bf16_row.hip -- the row, scalar and table kernels for bfloat16 storage
// (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_ROW_ENTRY_POINTS(, bf16_t)
}  // namespace rope
