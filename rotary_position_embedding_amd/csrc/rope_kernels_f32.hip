// rope_kernels_f32.hip -- the kernels for float32 storage (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_TYPE_ENTRY_POINTS(, float)
}  // namespace rope
