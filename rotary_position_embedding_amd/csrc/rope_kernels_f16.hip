// rope_kernels_f16.hip -- the kernels for float16 storage (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_TYPE_ENTRY_POINTS(, half_t)
}  // namespace rope
