// Library-wide entry points (version, status strings, sizes), host helpers,
// and the prefix-sum / fill kernels used by several stages.
#include <math.h>

#include <algorithm>

#include "internal.h"

namespace gs {

ShConsts sh_constants()
{
    ShConsts k;
    k.c0 = (float)(1.0 / (2.0 * sqrt(M_PI)));
    k.c1 = (float)sqrt(3.0 / (4.0 * M_PI));
    k.c2a = (float)(0.5 * sqrt(15.0 / M_PI));
    k.c2b = (float)(0.25 * sqrt(5.0 / M_PI));
    k.c2c = (float)(0.25 * sqrt(15.0 / M_PI));
    k.c3a = (float)(0.25 * sqrt(35.0 / (2.0 * M_PI)));
    k.c3b = (float)(0.5 * sqrt(105.0 / M_PI));
    k.c3c = (float)(0.25 * sqrt(21.0 / (2.0 * M_PI)));
    k.c3d = (float)(0.25 * sqrt(7.0 / M_PI));
    k.c3e = (float)(0.25 * sqrt(105.0 / M_PI));
    return k;
}

bool make_dev_cameras(const gs_camera* cams, int32_t n_views, DevCameras& out)
{
#pragma clang fp contract(off)
    if (!cams || n_views < 1 || n_views > GS_MAX_VIEWS) return false;
    const int32_t W = cams[0].width, H = cams[0].height;
    if (W <= 0 || H <= 0) return false;
    out.n_views = n_views;
    out.width = W;
    out.height = H;
    out.tiles_x = (W + GS_TILE - 1) / GS_TILE;
    out.tiles_y = (H + GS_TILE - 1) / GS_TILE;
    if (out.tiles_x > 65535 || out.tiles_y > 65535) return false;  // rectangles are uint16
    const int64_t tpv = (int64_t)out.tiles_x * out.tiles_y;
    if (tpv * n_views >= ((int64_t)1 << 31)) return false;
    out.tiles_per_view = (int32_t)tpv;
    for (int v = 0; v < n_views; ++v) {
        const gs_camera& c = cams[v];
        if (c.width != W || c.height != H) return false;
        if (!(c.fx > 0.f) || !(c.fy > 0.f)) return false;
        DevCamera& d = out.c[v];
        for (int i = 0; i < 9; ++i) d.R[i] = c.R[i];
        for (int i = 0; i < 3; ++i) d.t[i] = c.t[i];
        d.fx = c.fx; d.fy = c.fy; d.cx = c.cx; d.cy = c.cy;
        d.near_plane = c.near_plane;
        d.far_plane = c.far_plane;
        // fp32, fixed order: 1.3 x tan(half field of view)
        const float hw = 0.5f * (float)W, hh = 0.5f * (float)H;
        d.limx = 1.3f * (hw / c.fx);
        d.limy = 1.3f * (hh / c.fy);
        // camera centre -R^T t, fp32, fixed order
        d.ccx = -((c.R[0] * c.t[0] + c.R[3] * c.t[1]) + c.R[6] * c.t[2]);
        d.ccy = -((c.R[1] * c.t[0] + c.R[4] * c.t[1]) + c.R[7] * c.t[2]);
        d.ccz = -((c.R[2] * c.t[0] + c.R[5] * c.t[1]) + c.R[8] * c.t[2]);
    }
    return true;
}

// ---------------------------------------------------------------------------
// Reduce-then-scan prefix sum: 4096 items per block.
// ---------------------------------------------------------------------------
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 16;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;

size_t scan_workspace_bytes(uint64_t count)
{
    const uint64_t nb = (count + SCAN_TILE - 1) / SCAN_TILE;
    return (size_t)(nb + 1) * sizeof(uint64_t);
}

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x)
{
    const uint32_t lane = __lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T y = __shfl_up(x, off);
        if (lane >= (uint32_t)off) x += y;
    }
    return x;
}

// Exclusive scan of one value per thread over a 256-thread block.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T x, T* s_wave /*[4]*/, T& block_total)
{
    const uint32_t lane = __lane_id(), wave = threadIdx.x >> 6;
    const T inc = wave_inclusive_scan(x);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    T before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < SCAN_THREADS / 64; ++w) {
        const T t = s_wave[w];
        if (w < (int)wave) before += t;
        total += t;
    }
    __syncthreads();
    block_total = total;
    return before + inc - x;
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_reduce(const uint32_t* __restrict__ in, uint64_t count,
                                                              uint64_t* __restrict__ partial)
{
    __shared__ uint64_t s_wave[4];
    const uint64_t base = (uint64_t)blockIdx.x * SCAN_TILE;
    uint64_t sum = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        const uint64_t i = base + (uint64_t)k * SCAN_THREADS + threadIdx.x;
        if (i < count) sum += in[i];
    }
    uint64_t total;
    (void)block_exclusive_scan<uint64_t>(sum, s_wave, total);
    if (threadIdx.x == 0) partial[blockIdx.x] = total;
}

// One block: exclusive scan of the per-block totals, in place; total out.
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_partials(uint64_t* __restrict__ partial, uint64_t nb,
                                                                uint32_t* __restrict__ out_last,
                                                                uint64_t* __restrict__ total_out)
{
    __shared__ uint64_t s_wave[4];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nb; base += SCAN_THREADS) {
        const uint64_t i = base + threadIdx.x;
        const uint64_t x = i < nb ? partial[i] : 0;
        uint64_t chunk;
        const uint64_t ex = block_exclusive_scan<uint64_t>(x, s_wave, chunk);
        if (i < nb) partial[i] = carry + ex;
        carry += chunk;
    }
    if (threadIdx.x == 0) {
        *out_last = (uint32_t)carry;
        if (total_out) *total_out = carry;
    }
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_down(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                            uint64_t count, const uint64_t* __restrict__ partial)
{
    __shared__ uint32_t s_items[SCAN_TILE];
    __shared__ uint64_t s_wave[4];
    const uint64_t base = (uint64_t)blockIdx.x * SCAN_TILE;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        const uint64_t i = base + (uint64_t)k * SCAN_THREADS + threadIdx.x;
        s_items[k * SCAN_THREADS + threadIdx.x] = i < count ? in[i] : 0u;
    }
    __syncthreads();
    uint32_t v[SCAN_ITEMS];
    uint64_t sum = 0;
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        v[k] = s_items[threadIdx.x * SCAN_ITEMS + k];
        sum += v[k];
    }
    uint64_t tot;
    uint64_t run = partial[blockIdx.x] + block_exclusive_scan<uint64_t>(sum, s_wave, tot);
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        s_items[threadIdx.x * SCAN_ITEMS + k] = (uint32_t)run;
        run += v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SCAN_ITEMS; ++k) {
        const uint64_t i = base + (uint64_t)k * SCAN_THREADS + threadIdx.x;
        if (i < count) out[i] = s_items[k * SCAN_THREADS + threadIdx.x];
    }
}

hipError_t scan_u32(const uint32_t* in, uint32_t* out, uint64_t count, uint64_t* total, void* ws,
                    hipStream_t stream)
{
    uint64_t* partial = (uint64_t*)ws;
    const uint64_t nb = (count + SCAN_TILE - 1) / SCAN_TILE;
    if (nb > 0) {
        hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, stream, in, count, partial);
    }
    hipLaunchKernelGGL(k_scan_partials, dim3(1), dim3(SCAN_THREADS), 0, stream, partial, nb, out + count, total);
    if (nb > 0) {
        hipLaunchKernelGGL(k_scan_down, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, stream, in, out, count,
                           (const uint64_t*)partial);
    }
    return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t* __restrict__ dst, uint64_t count, uint32_t value)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) dst[i] = value;
}

hipError_t fill_u32(uint32_t* dst, uint64_t count, uint32_t value, hipStream_t stream)
{
    if (count == 0) return hipSuccess;
    uint64_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, stream, dst, count, value);
    return hipGetLastError();
}

// A plain device copy, 16-byte vectors, four in flight per thread per round
// (a grid-stride loop over a grid that fills the chip). It moves exactly
// 2 x bytes of device memory and nothing else, which makes it the reference
// for the achievable HBM bandwidth and for scaling the profiler's traffic
// counters.
constexpr int COPY_THREADS = 256;

__global__ __launch_bounds__(COPY_THREADS) void k_stream_copy(float4* __restrict__ dst, const float4* __restrict__ src,
                                                             uint64_t n4)
{
    const uint64_t stride = (uint64_t)gridDim.x * COPY_THREADS;
    uint64_t i = (uint64_t)blockIdx.x * COPY_THREADS + threadIdx.x;
    // streaming (nontemporal) loads and stores: each byte is touched once
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f* s4 = (const v4f*)src;
    v4f* d4 = (v4f*)dst;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const v4f a = __builtin_nontemporal_load(s4 + i), b = __builtin_nontemporal_load(s4 + i + stride),
                  c = __builtin_nontemporal_load(s4 + i + 2 * stride), d = __builtin_nontemporal_load(s4 + i + 3 * stride);
        __builtin_nontemporal_store(a, d4 + i);
        __builtin_nontemporal_store(b, d4 + i + stride);
        __builtin_nontemporal_store(c, d4 + i + 2 * stride);
        __builtin_nontemporal_store(d, d4 + i + 3 * stride);
    }
    for (; i < n4; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + i), d4 + i);
}

}  // namespace gs

extern "C" {

int gs_abi_version(void) { return GS_ABI_VERSION; }

const char* gs_status_string(gs_status s)
{
    switch (s) {
        case GS_OK: return "ok";
        case GS_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GS_ERR_CAPACITY: return "capacity exceeded";
        case GS_ERR_HIP: return "HIP runtime error";
        case GS_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

int gs_param_rows(int32_t sh_degree)
{
    if (sh_degree < 0 || sh_degree > 3) return -1;
    return 11 + 3 * (sh_degree + 1) * (sh_degree + 1);
}

int32_t gs_tiles_x(int32_t width) { return width <= 0 ? 0 : (width + GS_TILE - 1) / GS_TILE; }
int32_t gs_tiles_y(int32_t height) { return height <= 0 ? 0 : (height + GS_TILE - 1) / GS_TILE; }

int32_t gs_sort_end_bit(int32_t n_views, int64_t tiles_per_view)
{
    const int64_t ids = (int64_t)n_views * tiles_per_view;
    int bits = 0;
    while (bits < 31 && ((int64_t)1 << bits) < ids) ++bits;
    return 32 + bits;
}

size_t gs_preprocess_workspace_bytes(int64_t n, int32_t n_views)
{
    if (n < 0 || n_views < 1) return 0;
    // the scan of the counts, or (without offsets) the wave sums
    return std::max<size_t>(gs::scan_workspace_bytes((uint64_t)n * (uint64_t)n_views), (size_t)((n + 63) / 64) * 4);
}

gs_status gs_stream_copy(void* dst, const void* src, uint64_t bytes, void* stream)
{
    if (bytes == 0) return GS_OK;
    if (!dst || !src || (bytes & 15u) || ((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u))
        return GS_ERR_INVALID_ARGUMENT;
    const uint64_t n4 = bytes / 16u;
    const uint64_t blocks = (n4 + gs::COPY_THREADS - 1) / gs::COPY_THREADS;
    const unsigned grid = (unsigned)(blocks < 256u * 32u ? blocks : 256u * 32u);  // 32 workgroups per CU at most
    hipLaunchKernelGGL(gs::k_stream_copy, dim3(grid), dim3(gs::COPY_THREADS), 0, (hipStream_t)stream, (float4*)dst,
                       (const float4*)src, n4);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
