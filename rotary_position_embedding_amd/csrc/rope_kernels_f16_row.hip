// rope_kernels_f16_row.hip -- the row, scalar and table kernels for float16 storage
// (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_ROW_ENTRY_POINTS(, half_t)
}  // namespace rope
