// gs_tile_masks: for every entry of the per-tile lists, the 16-bit mask of
// the tile's 4x4-pixel sub-blocks that the entry's alpha >= 1/255 region can
// touch (tile_mask16 in raster_common.h). The blending rule of the method
// (skip an entry wherever its alpha is below 1/255; 3DGS, reference [10] of
// "A Scalable PyTorch Abstraction for Multi-GPU Gaussian Splatting") makes
// such a sub-block's pairs no-ops, so the raster kernels drop them before
// gathering a record; computing the mask once per list entry spares each
// quarter of a tile, forward and backward, the ellipse test and the record
// gathers of entries that miss it.
//
// Two kernels: the tile of every list position (one wavefront per tile
// storing its index over the tile's range; positions outside every range
// keep -1), then one thread per list position, so that a tile with thousands
// of entries is spread over the whole chip.
#include "raster_common.h"

namespace gs {

constexpr int TM_THREADS = 256;

__global__ __launch_bounds__(TM_THREADS) void k_tile_of(const uint32_t* __restrict__ ranges, int64_t n_tiles,
                                                        int32_t* __restrict__ tile_of)
{
    const int64_t tl = (int64_t)blockIdx.x * (TM_THREADS / 64) + (threadIdx.x >> 6);
    if (tl >= n_tiles) return;
    const uint2 rg = *(const uint2*)(ranges + 2 * tl);
    for (uint32_t p = rg.x + (threadIdx.x & 63u); p < rg.y; p += 64u) tile_of[p] = (int32_t)tl;
}

__global__ __launch_bounds__(TM_THREADS) void k_tile_masks(const float* __restrict__ rec, int64_t n,
                                                           const int32_t* __restrict__ tile_of,
                                                           const uint32_t* __restrict__ vals, uint64_t capacity,
                                                           int W, int H, int TX, int T, uint16_t* __restrict__ masks)
{
    const uint64_t p = (uint64_t)blockIdx.x * TM_THREADS + threadIdx.x;
    if (p >= capacity) return;
    const int32_t tl = tile_of[p];
    if (tl < 0) return;
    const int view = tl / T;
    const int tile = tl - view * T;
    const int ty = tile / TX, tx = tile - ty * TX;
    Entry E;
    E.valid = true;
    E.gid = vals[p];
    gather_record(E, rec + (int64_t)view * n * GS_REC_FLOATS, n);
    masks[p] = (uint16_t)tile_mask16(E, tx * 16, ty * 16, W, H);
}

}  // namespace gs

using namespace gs;

extern "C" {

size_t gs_tile_masks_workspace_bytes(uint64_t capacity) { return (size_t)capacity * sizeof(int32_t); }

gs_status gs_tile_masks(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                        uint64_t capacity, const gs_camera* cams, int32_t n_views, uint16_t* masks, void* ws,
                        size_t ws_bytes, void* stream)
{
    if (n < 0 || !ranges) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && capacity > 0 && (!rec || !vals || !masks || !ws)) return GS_ERR_INVALID_ARGUMENT;
    if (capacity >= ((uint64_t)1 << 32) || ws_bytes < gs_tile_masks_workspace_bytes(capacity))
        return GS_ERR_INVALID_ARGUMENT;
    DevCameras dc;
    if (!make_dev_cameras(cams, n_views, dc)) return GS_ERR_INVALID_ARGUMENT;
    if (n == 0 || capacity == 0) return GS_OK;
    const int64_t n_tiles = (int64_t)n_views * dc.tiles_per_view;
    if (n_tiles >= ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    int32_t* tile_of = (int32_t*)ws;
    if (fill_u32((uint32_t*)tile_of, capacity, 0xffffffffu, s) != hipSuccess) return GS_ERR_HIP;
    hipLaunchKernelGGL(k_tile_of, dim3((unsigned)((n_tiles + TM_THREADS / 64 - 1) / (TM_THREADS / 64))),
                       dim3(TM_THREADS), 0, s, ranges, n_tiles, tile_of);
    hipLaunchKernelGGL(k_tile_masks, dim3(grid_for(capacity, TM_THREADS)), dim3(TM_THREADS), 0, s, rec, n, tile_of,
                       vals, capacity, dc.width, dc.height, dc.tiles_x, dc.tiles_per_view, masks);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
