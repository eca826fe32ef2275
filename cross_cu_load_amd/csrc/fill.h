// Launch of the output fill for units without pieces (empty sequences).
#pragma once

#include <hip/hip_runtime.h>

#include "launch.h"

namespace cc {
// out = 0, lse = -inf for every unit whose unit_nsplit is 0, on stream s
// (records a.ev_start / a.ev_stop around the launch when set).
hipError_t launch_empty_units(const DecodeArgs& a, hipStream_t s);
}  // namespace cc
