// gs_rasterize_bwd: back-to-front gradients of the alpha compositing to the
// 2D quantities of every (view, Gaussian) (backward rasterization of the
// ByteSplat abstract). The walk over a quarter's list, its two phases and the
// derivatives are in raster_bwd.h; this kernel reads each pixel's T_final,
// n_contrib and dL/dimage from the forward pass.
#include "raster_bwd.h"

namespace gs {

__global__ __launch_bounds__(RW_THREADS) void k_raster_bwd(const float* __restrict__ rec, int64_t n,
                                                           const uint32_t* __restrict__ ranges,
                                                           const uint32_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ masks, uint32_t cap, int W,
                                                           int H, int TX, int T, int row0, float bg0, float bg1, float bg2,
                                                           const float* __restrict__ T_final,
                                                           const int32_t* __restrict__ n_contrib,
                                                           const float* __restrict__ dL_dimage,
                                                           float* __restrict__ grad2d)
{
#pragma clang fp contract(off)
    const QuarterCtx t = quarter_ctx(W, H, TX, T, row0);
    if (t.empty) return;
    const int64_t HW = (int64_t)H * W;
    const int64_t pix = (int64_t)t.j * W + t.i;
    int32_t my_last = 0;
    float Tr = 1.f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
    if (t.inside) {
        my_last = n_contrib[(int64_t)t.view * HW + pix];
        Tr = T_final[(int64_t)t.view * HW + pix];
        const float* gimg = dL_dimage + (int64_t)t.view * 3 * HW + pix;
        g0 = gimg[0];
        g1 = gimg[HW];
        g2 = gimg[2 * HW];
    }
    __shared__ BwdLds lds;
    raster_bwd_walk(lds, t, my_last, Tr, g0, g1, g2, bg0, bg1, bg2, rec, n, ranges, vals, masks, cap, grad2d);
}

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_rasterize_bwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, const float* T_final,
                           const int32_t* n_contrib, const float* dL_dimage, float* grad2d, int32_t accumulate,
                           void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, a))
        return GS_ERR_INVALID_ARGUMENT;
    if (!T_final || !n_contrib || !dL_dimage || (n > 0 && !grad2d)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate && n > 0) {
        if (fill_u32((uint32_t*)grad2d, (uint64_t)n_views * GS_GRAD2D_ROWS * (uint64_t)n, 0u, s) != hipSuccess)
            return GS_ERR_HIP;
    }
    hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, s, rec, n, ranges, vals,
                       masks, a.cap, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2], T_final,
                       n_contrib, dL_dimage, grad2d);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
