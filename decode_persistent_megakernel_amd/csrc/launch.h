// Host-side launchers of the device code (internal to libmk).
#pragma once

#include <hip/hip_runtime_api.h>

#include "device.h"

namespace mk {

hipError_t set_lds_limit(int bytes);
hipError_t persistent_occupancy(int lds, int* blocks_per_cu);
// mfma: the matrix-core variant (batch up to kMfmaCols), else the vector one (batch up to kMaxCols)
hipError_t launch_persistent(const Params& P, int grid, int lds, bool mfma, hipStream_t s);
hipError_t launch_op(const Params& P, int first, int count, int lds, bool mfma, hipStream_t s);
// Static workspace of mk_generate_noalloc: resolve the device address of the
// array on `dev` (which must be current) once; later calls return at once.
hipError_t noalloc_scratch_init(int dev);
// The address resolved for `dev`, or nullptr before noalloc_scratch_init.
void* noalloc_scratch(int dev);
hipError_t launch_fill_zero(uint32_t* p, size_t words, hipStream_t s);
hipError_t launch_pack(const PackJob* jobs, int n_jobs, const PackSrc* src, uint8_t* dst, int G, int D, int L,
                       bool mfma, hipStream_t s);

}  // namespace mk
