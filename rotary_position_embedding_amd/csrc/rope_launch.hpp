// rope_launch.hpp -- entry points of the HIP side (rope_kernels.hip).
#pragma once

#include "rope_plan.hpp"

namespace rope {

// Enqueue the kernels of a validated plan on `stream` (a hipStream_t).
int launch_plan(const Plan& plan, void* stream);
int launch_inv_freq(float* inv_freq, int64_t half, double base, void* stream);
int launch_cos_sin_cache(const TablePlan& table, void* stream);

}  // namespace rope
