// Host-side helpers shared by the entry points (not exported).
#pragma once

#include "common.h"

namespace gs {

// Validates the cameras (count, equal sizes, positive focal lengths) and
// converts them to the kernels' form (guard band, camera centre). Returns
// false on invalid input.
bool make_dev_cameras(const gs_camera* cams, int32_t n_views, DevCameras& out);

// fp32 values of the real SH constants, from their closed forms in fp64.
ShConsts sh_constants();

// Exclusive prefix sum of `count` uint32 values into `out` (may alias `in`),
// with out[count] = low 32 bits of the total and *total (if not null) = the
// 64-bit total. Workspace: scan_workspace_bytes(count).
size_t scan_workspace_bytes(uint64_t count);
hipError_t scan_u32(const uint32_t* in, uint32_t* out, uint64_t count, uint64_t* total, void* ws,
                    hipStream_t stream);

// Fill `count` uint32 with `value` (a kernel, so it is safe inside graphs).
hipError_t fill_u32(uint32_t* dst, uint64_t count, uint32_t value, hipStream_t stream);

// *loss (+)= scale * sum of `count` per-quarter partial sums of |I - I*|
// (the L1 loss of the raster kernels): overwritten unless `accumulate`; the
// same bits on every run. The workspace holds, after the partials, the
// reduction's tail (LOSS_TAIL_BYTES, raster_fwd.h), whose counter the raster
// kernel that wrote the partials has reset.
hipError_t loss_from_partials(const double* partial, int64_t count, double scale, double* loss, bool accumulate,
                              hipStream_t stream);

inline unsigned grid_for(uint64_t items, unsigned per_block)
{
    return (unsigned)((items + per_block - 1) / per_block);
}

}  // namespace gs
