// rope_kernels_f16.hip -- the vector kernel for float16 storage (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_VEC_ENTRY_POINTS(, half_t)
}  // namespace rope
