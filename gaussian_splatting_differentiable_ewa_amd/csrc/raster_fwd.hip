// gs_rasterize_fwd: per-tile alpha compositing over the sorted intersection
// lists (forward rasterization of the ByteSplat abstract). The walk over a
// quarter's list, its work decomposition and per-pair arithmetic are in
// raster_fwd.h.
#include "raster_fwd.h"

namespace gs {

// The L1 loss fused at the end (L1 = true): each lane reads its pixel's
// target, writes dL/dimage = scale sign(I - I*) and the wave's sum of |I - I*|
// goes to partial[block] (0 for quarters outside the image); image may then
// be null.
template <bool L1>
__device__ __forceinline__ void raster_fwd_body(const float* __restrict__ rec, int64_t n,
                                                const uint32_t* __restrict__ ranges,
                                                const uint32_t* __restrict__ vals,
                                                const uint16_t* __restrict__ masks, uint32_t cap, int W, int H,
                                                int TX, int T, int row0, float bg0, float bg1, float bg2, float* __restrict__ image,
                                                float* __restrict__ T_final, int32_t* __restrict__ n_contrib,
                                                const float* __restrict__ target, float scale,
                                                float* __restrict__ dL, double* __restrict__ partial)
{
#pragma clang fp contract(off)
    __shared__ FwdLds lds;
    if (L1 && blockIdx.x == 0 && threadIdx.x == 0) *loss_counter(partial, gridDim.x) = 0u;
    const QuarterCtx t = quarter_ctx(W, H, TX, T, row0);
    if (t.empty) {
        if (L1 && t.lane == 0) partial[blockIdx.x] = 0.0;
        return;
    }
    const int64_t HW = (int64_t)H * W;
    const int64_t pix = (int64_t)t.j * W + t.i;
    const int64_t o = (int64_t)t.view * 3 * HW + pix;
    // the target of this lane's pixel, requested now and used at the end
    float tg0 = 0.f, tg1 = 0.f, tg2 = 0.f;
    if (L1 && t.inside) {
        tg0 = target[o];
        tg1 = target[o + HW];
        tg2 = target[o + 2 * HW];
    }
    const FwdPixel P = raster_fwd_walk(lds, t, rec, n, ranges, vals, masks, cap);
    float ad = 0.f;  // |I - I*| summed over the channels
    if (t.inside) {
        const float i0 = P.C0 + P.Tr * bg0, i1 = P.C1 + P.Tr * bg1, i2 = P.C2 + P.Tr * bg2;
        if (!L1 || image) {
            image[o] = i0;
            image[o + HW] = i1;
            image[o + 2 * HW] = i2;
        }
        T_final[(int64_t)t.view * HW + pix] = P.Tr;
        n_contrib[(int64_t)t.view * HW + pix] = P.last;
        if (L1) {
            const float d0 = i0 - tg0, d1 = i1 - tg1, d2 = i2 - tg2;
            dL[o] = l1_grad(d0, scale);
            dL[o + HW] = l1_grad(d1, scale);
            dL[o + 2 * HW] = l1_grad(d2, scale);
            ad = (fabsf(d0) + fabsf(d1)) + fabsf(d2);
        }
    }
    if (L1) loss_partial(ad, t.lane, partial);
}

__global__ __launch_bounds__(RW_THREADS) void k_raster_fwd(const float* __restrict__ rec, int64_t n,
                                                           const uint32_t* __restrict__ ranges,
                                                           const uint32_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ masks, uint32_t cap, int W,
                                                           int H, int TX, int T, int row0, float bg0, float bg1,
                                                           float bg2, float* __restrict__ image,
                                                           float* __restrict__ T_final, int32_t* __restrict__ n_contrib)
{
    raster_fwd_body<false>(rec, n, ranges, vals, masks, cap, W, H, TX, T, row0, bg0, bg1, bg2, image, T_final, n_contrib, nullptr, 0.f,
                           nullptr, nullptr);
}

__global__ __launch_bounds__(RW_THREADS) void k_raster_fwd_l1(const float* __restrict__ rec, int64_t n,
                                                              const uint32_t* __restrict__ ranges,
                                                              const uint32_t* __restrict__ vals,
                                                              const uint16_t* __restrict__ masks, uint32_t cap, int W,
                                                              int H, int TX, int T, int row0, float bg0, float bg1,
                                                              float bg2, float* __restrict__ image,
                                                              float* __restrict__ T_final, int32_t* __restrict__ n_contrib,
                                                              const float* __restrict__ target, float scale,
                                                              float* __restrict__ dL, double* __restrict__ partial)
{
    raster_fwd_body<true>(rec, n, ranges, vals, masks, cap, W, H, TX, T, row0, bg0, bg1, bg2, image, T_final, n_contrib, target, scale,
                          dL, partial);
}

// The sum of 256 values, one per thread, in a fixed order (every thread
// returns it).
__device__ __forceinline__ double block_sum_256(double v, double* s_w)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

// loss (+)= scale * sum of the per-quarter partial sums, the same bits on
// every run: each workgroup sums a contiguous slice in a fixed order and
// stores it; the workgroup that arrives last (the arrival counter after the
// sums) adds the workgroups' sums in index order and writes the loss.
__global__ __launch_bounds__(256) void k_loss_partials(const double* __restrict__ partial, int64_t count,
                                                       double scale, double* __restrict__ loss, int accumulate)
{
    __shared__ double s_w[4], s_w2[4];
    __shared__ int s_last;
    double* bsum = const_cast<double*>(partial) + count;
    uint32_t* counter = loss_counter(const_cast<double*>(partial), count);
    const int64_t per = (count + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(count, b0 + per);
    double acc = 0.0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 256) acc += partial[i];
    const double mine = block_sum_256(acc, s_w);
    if (threadIdx.x == 0) {
        __hip_atomic_store(bsum + blockIdx.x, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = before == gridDim.x - 1u;
    }
    __syncthreads();
    if (!s_last) return;
    const double v = threadIdx.x < gridDim.x
                         ? __hip_atomic_load(bsum + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.0;
    const double total = block_sum_256(v, s_w2);
    if (threadIdx.x == 0) {
        *loss = accumulate ? *loss + total * scale : total * scale;
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The raster passes' exponential, element-wise (for checks of its error).
__global__ __launch_bounds__(256) void k_raster_exp(const float* __restrict__ x, float* __restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = exp_fast(x[i]);
}

hipError_t loss_from_partials(const double* partial, int64_t count, double scale, double* loss, bool accumulate,
                              hipStream_t stream)
{
    const unsigned red_blocks = (unsigned)(count < LOSS_BLOCKS * 64 ? (count + 63) / 64 : LOSS_BLOCKS);
    hipLaunchKernelGGL(k_loss_partials, dim3(red_blocks), dim3(256), 0, stream, partial, count, scale, loss,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace gs

using namespace gs;

extern "C" {

size_t gs_rasterize_fwd_l1_workspace_bytes(int32_t n_views, int32_t width, int32_t height)
{
    if (n_views < 1 || n_views > GS_MAX_VIEWS || width <= 0 || height <= 0) return 0;
    const int64_t quarters = (int64_t)n_views * gs_tiles_x(width) * gs_tiles_y(height) * 4;
    return (size_t)quarters * sizeof(double) + LOSS_TAIL_BYTES;
}

gs_status gs_rasterize_fwd_l1(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                              const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views, int32_t row0,
                              int32_t rows, const float* bg, const float* target,
                              float scale, float* image, float* T_final, int32_t* n_contrib, float* dL_dimage,
                              double* loss, int32_t accumulate, void* ws, size_t ws_bytes, void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, a))
        return GS_ERR_INVALID_ARGUMENT;
    if (!T_final || !n_contrib || !target || !dL_dimage || !loss || !ws) return GS_ERR_INVALID_ARGUMENT;
    if (ws_bytes < (size_t)a.n_blocks * sizeof(double) + LOSS_TAIL_BYTES) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    double* partial = (double*)ws;
    hipLaunchKernelGGL(k_raster_fwd_l1, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, s, rec, n, ranges, vals,
                       masks, a.cap, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2], image, T_final,
                       n_contrib, target, scale, dL_dimage, partial);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    return loss_from_partials(partial, a.n_blocks, (double)scale, loss, accumulate != 0, s) == hipSuccess ? GS_OK
                                                                                                           : GS_ERR_HIP;
}

gs_status gs_rasterize_fwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, float* image, float* T_final,
                           int32_t* n_contrib, void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, a))
        return GS_ERR_INVALID_ARGUMENT;
    if (!image || !T_final || !n_contrib) return GS_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(k_raster_fwd, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, (hipStream_t)stream, rec, n,
                       ranges, vals, masks, a.cap, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2],
                       image, T_final, n_contrib);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_raster_exp(const float* x, float* y, int64_t n, void* stream)
{
    if (n < 0 || (n > 0 && (!x || !y)) || n >= ((int64_t)1 << 40)) return GS_ERR_INVALID_ARGUMENT;
    if (n == 0) return GS_OK;
    hipLaunchKernelGGL(k_raster_exp, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, x, y, n);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
