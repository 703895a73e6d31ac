// Host-side launchers of the device code (internal to libmk).
#pragma once

#include <hip/hip_runtime_api.h>

#include "device.h"

namespace mk {

hipError_t set_lds_limit(int bytes);
hipError_t persistent_occupancy(int lds, int* blocks_per_cu);
hipError_t launch_persistent(const Params& P, int grid, int lds, hipStream_t s);
hipError_t launch_op(const Params& P, int first, int count, int lds, hipStream_t s);
hipError_t launch_pack(const PackJob* jobs, int n_jobs, const PackSrc* src, uint8_t* dst, int G, int D, int L,
                       hipStream_t s);

}  // namespace mk
