// Launcher of the device-side input check (check.hip), used by the host API.
// Internal to the library.
#pragma once

#include "launch.h"

namespace fp8pa {

// Check of a decode call's device-side inputs into `report` (int32[16]):
// a reset of the report, then one workgroup per request and, for sparse
// calls, one per query row.  Returns hipSuccess or the launch error.
hipError_t launch_check(const DecodeArgs& a, int32_t* report, hipStream_t stream);

}  // namespace fp8pa
