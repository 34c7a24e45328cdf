// rope_kernels_bf16.hip -- the vector kernel for bfloat16 storage (see rope_device.hpp).
#include "rope_device.hpp"

namespace rope {
ROPE_VEC_ENTRY_POINTS(, bf16_t)
}  // namespace rope
