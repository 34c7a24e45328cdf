// rope_kernels_f32.hip -- the vector kernel for float32 storage (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_VEC_ENTRY_POINTS(, float)
}  // namespace rope
