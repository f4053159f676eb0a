// gs_window_gaussians: per view, the Gaussians whose tile rectangle meets a
// window of tile rows, in index order -- the input of gs_tile_lists when an
// image is processed window by window so that the intersection lists need
// only hold one window (the per-tile intersection lists are what runs out of
// memory first at 4K: "AMD ROCm team open-sources distributed 3D Gaussian
// Splatting training", section "Distributed training architecture and memory
// scaling"). Binning a window then reads only its own Gaussians.
//
// gs_seen_gaussians: likewise, the Gaussians some view sees (the set whose
// gradients a compact backward writes).
//
// An order-preserving compaction: k_window_count counts each 256-Gaussian
// block's members (one ballot per wave), the counts of all views' blocks are
// scanned, and k_window_write writes each member at its block's offset plus
// its rank among the block's members.
#include "internal.h"

namespace gs {

constexpr int WIN_THREADS = 256;

__device__ __forceinline__ bool window_member(const uint16_t* __restrict__ rect, int64_t idx, int32_t row0,
                                              int32_t row1)
{
    const uint2 rr = *(const uint2*)(rect + 4 * idx);
    const int32_t x0 = (int32_t)(rr.x & 0xffffu), y0 = (int32_t)(rr.x >> 16);
    const int32_t x1 = (int32_t)(rr.y & 0xffffu), y1 = (int32_t)(rr.y >> 16);
    return x1 > x0 && y1 > y0 && y0 < row1 && y1 > row0;
}

// block b of view v (blocks_per_view blocks of 256 Gaussians each)
__global__ __launch_bounds__(WIN_THREADS) void k_window_count(const uint16_t* __restrict__ rect, int64_t n,
                                                              int64_t blocks_per_view, int32_t row0, int32_t row1,
                                                              uint32_t* __restrict__ counts)
{
    __shared__ uint32_t s_cnt[WIN_THREADS / 64];
    const int64_t v = blockIdx.x / blocks_per_view, b = blockIdx.x - v * blocks_per_view;
    const int64_t g = b * WIN_THREADS + threadIdx.x;
    const bool in = g < n && window_member(rect, v * n + g, row0, row1);
    const uint64_t m = ballot(in);
    if ((threadIdx.x & 63u) == 0u) s_cnt[threadIdx.x >> 6] = (uint32_t)__popcll(m);
    __syncthreads();
    if (threadIdx.x == 0) counts[blockIdx.x] = (s_cnt[0] + s_cnt[1]) + (s_cnt[2] + s_cnt[3]);
}

__global__ __launch_bounds__(WIN_THREADS) void k_window_write(const uint16_t* __restrict__ rect, int64_t n,
                                                              int64_t blocks_per_view, int32_t row0, int32_t row1,
                                                              const uint32_t* __restrict__ offsets,
                                                              uint32_t* __restrict__ gauss,
                                                              uint32_t* __restrict__ view_off, int32_t n_views)
{
    __shared__ uint32_t s_cnt[WIN_THREADS / 64];
    const int64_t v = blockIdx.x / blocks_per_view, b = blockIdx.x - v * blocks_per_view;
    const int64_t g = b * WIN_THREADS + threadIdx.x;
    const bool in = g < n && window_member(rect, v * n + g, row0, row1);
    const uint64_t m = ballot(in);
    const uint32_t w = threadIdx.x >> 6;
    if ((threadIdx.x & 63u) == 0u) s_cnt[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = offsets[blockIdx.x];
    for (uint32_t k = 0; k < w; ++k) before += s_cnt[k];
    if (in) gauss[before + mask_rank(m)] = (uint32_t)g;
    // each view's segment starts at the offset of its first block; the last
    // block of the last view writes the total
    if (threadIdx.x == 0 && b == 0) view_off[v] = offsets[blockIdx.x];
    if (threadIdx.x == 0 && blockIdx.x == (int64_t)n_views * blocks_per_view - 1)
        view_off[n_views] = offsets[blockIdx.x + 1];
}

// gs_seen_gaussians: the same compaction over the Gaussians whose rectangle is
// non-empty in some view (one list for all views)
__device__ __forceinline__ bool seen_in_any(const uint16_t* __restrict__ rect, int64_t n, int32_t n_views, int64_t g)
{
    bool seen = false;
    for (int v = 0; v < n_views; ++v) {
        const uint2 rr = *(const uint2*)(rect + 4 * ((int64_t)v * n + g));
        seen = seen || ((rr.y & 0xffffu) > (rr.x & 0xffffu) && (rr.y >> 16) > (rr.x >> 16));
    }
    return seen;
}

__global__ __launch_bounds__(WIN_THREADS) void k_seen_count(const uint16_t* __restrict__ rect, int64_t n,
                                                            int32_t n_views, uint32_t* __restrict__ counts)
{
    __shared__ uint32_t s_cnt[WIN_THREADS / 64];
    const int64_t g = (int64_t)blockIdx.x * WIN_THREADS + threadIdx.x;
    const bool in = g < n && seen_in_any(rect, n, n_views, g);
    const uint64_t m = ballot(in);
    if ((threadIdx.x & 63u) == 0u) s_cnt[threadIdx.x >> 6] = (uint32_t)__popcll(m);
    __syncthreads();
    if (threadIdx.x == 0) counts[blockIdx.x] = (s_cnt[0] + s_cnt[1]) + (s_cnt[2] + s_cnt[3]);
}

__global__ __launch_bounds__(WIN_THREADS) void k_seen_write(const uint16_t* __restrict__ rect, int64_t n,
                                                            int32_t n_views, const uint32_t* __restrict__ offsets,
                                                            uint32_t* __restrict__ list, uint32_t* __restrict__ count)
{
    __shared__ uint32_t s_cnt[WIN_THREADS / 64];
    const int64_t g = (int64_t)blockIdx.x * WIN_THREADS + threadIdx.x;
    const bool in = g < n && seen_in_any(rect, n, n_views, g);
    const uint64_t m = ballot(in);
    const uint32_t w = threadIdx.x >> 6;
    if ((threadIdx.x & 63u) == 0u) s_cnt[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = offsets[blockIdx.x];
    for (uint32_t k = 0; k < w; ++k) before += s_cnt[k];
    if (in) list[before + mask_rank(m)] = (uint32_t)g;
    if (threadIdx.x == 0 && blockIdx.x == gridDim.x - 1) *count = offsets[blockIdx.x + 1];
}

}  // namespace gs

using namespace gs;

extern "C" {

size_t gs_window_gaussians_workspace_bytes(int64_t n, int32_t n_views)
{
    if (n < 0 || n_views < 1 || n_views > GS_MAX_VIEWS) return 0;
    const uint64_t blocks = (uint64_t)n_views * (uint64_t)((n + WIN_THREADS - 1) / WIN_THREADS);
    return (size_t)((blocks + 1) * 4 + 255) / 256 * 256 + scan_workspace_bytes(blocks);
}

gs_status gs_window_gaussians(const uint16_t* rect, int64_t n, int32_t n_views, int32_t height, int32_t row0,
                              int32_t rows, uint32_t* gauss, uint32_t* view_off, void* ws, size_t ws_bytes,
                              void* stream)
{
    if (n < 0 || n_views < 1 || n_views > GS_MAX_VIEWS || height <= 0) return GS_ERR_INVALID_ARGUMENT;
    if (row0 < 0 || rows < 1 || row0 + rows > gs_tiles_y(height)) return GS_ERR_INVALID_ARGUMENT;
    if (!view_off || !ws || (n > 0 && (!rect || !gauss))) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    if (ws_bytes < gs_window_gaussians_workspace_bytes(n, n_views)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    const int64_t bpv = (n + WIN_THREADS - 1) / WIN_THREADS;
    const uint64_t blocks = (uint64_t)n_views * (uint64_t)bpv;
    if (blocks == 0) return fill_u32(view_off, (uint64_t)n_views + 1, 0u, s) == hipSuccess ? GS_OK : GS_ERR_HIP;
    uint32_t* counts = (uint32_t*)ws;
    void* scan_ws = (char*)ws + ((blocks + 1) * 4 + 255) / 256 * 256;
    hipLaunchKernelGGL(k_window_count, dim3((unsigned)blocks), dim3(WIN_THREADS), 0, s, rect, n, bpv, row0,
                       row0 + rows, counts);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    if (scan_u32(counts, counts, blocks, nullptr, scan_ws, s) != hipSuccess) return GS_ERR_HIP;
    hipLaunchKernelGGL(k_window_write, dim3((unsigned)blocks), dim3(WIN_THREADS), 0, s, rect, n, bpv, row0,
                       row0 + rows, counts, gauss, view_off, n_views);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

size_t gs_seen_gaussians_workspace_bytes(int64_t n)
{
    if (n < 0) return 0;
    const uint64_t blocks = (uint64_t)((n + WIN_THREADS - 1) / WIN_THREADS);
    return (size_t)((blocks + 1) * 4 + 255) / 256 * 256 + scan_workspace_bytes(blocks);
}

gs_status gs_seen_gaussians(const uint16_t* rect, int64_t n, int32_t n_views, uint32_t* list, uint32_t* count,
                            void* ws, size_t ws_bytes, void* stream)
{
    if (n < 0 || n_views < 1 || n_views > GS_MAX_VIEWS) return GS_ERR_INVALID_ARGUMENT;
    if (!count || !ws || (n > 0 && (!rect || !list))) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    if (ws_bytes < gs_seen_gaussians_workspace_bytes(n)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    const uint64_t blocks = (uint64_t)((n + WIN_THREADS - 1) / WIN_THREADS);
    if (blocks == 0) return fill_u32(count, 1, 0u, s) == hipSuccess ? GS_OK : GS_ERR_HIP;
    uint32_t* counts = (uint32_t*)ws;
    void* scan_ws = (char*)ws + ((blocks + 1) * 4 + 255) / 256 * 256;
    hipLaunchKernelGGL(k_seen_count, dim3((unsigned)blocks), dim3(WIN_THREADS), 0, s, rect, n, n_views, counts);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    if (scan_u32(counts, counts, blocks, nullptr, scan_ws, s) != hipSuccess) return GS_ERR_HIP;
    hipLaunchKernelGGL(k_seen_write, dim3((unsigned)blocks), dim3(WIN_THREADS), 0, s, rect, n, n_views, counts,
                       list, count);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
