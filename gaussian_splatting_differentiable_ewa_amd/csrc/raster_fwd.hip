// gs_rasterize_fwd: per-tile alpha compositing over the sorted intersection
// lists (forward rasterization of the ByteSplat abstract; 16x16 pixel blocks
// of "On Scaling Up 3D Gaussian Splatting Training", answer (1); depth-sorted
// per-tile lists of the ROCm page, section "Distributed training architecture
// and memory scaling").
//
// Work decomposition (gfx950, wave64):
//   * one 64-lane workgroup per 8x8 quarter of a 16x16 tile, one lane per
//     pixel; the four quarters of a tile are independent wavefronts, so each
//     stops as soon as its own pixels are saturated and nothing waits at a
//     barrier;
//   * each 16-lane DPP row owns a 4x4 sub-block of the quarter and walks its
//     own list of entries;
//   * the tile's sorted list is read in batches of 64: each lane gathers one
//     entry's 48-byte record (the next batch's gathers are in flight while the
//     current batch is evaluated), computes the 4-bit mask of sub-blocks that
//     the region where the entry's alpha can reach 1/255 touches, and stages
//     it in LDS; each row compacts the entries of its bit (ballot + mbcnt,
//     list order kept);
//   * in the pixel loop every row reads its own next entry (an LDS broadcast
//     within the row), so one instruction stream advances four sub-blocks on
//     four different entries. An entry skipped by the mask has alpha < 1/255
//     at every pixel of the sub-block and would have been skipped anyway:
//     results are unchanged. Row lists hold record byte offsets and are
//     padded to the longest row's count with a slot of opacity 0 (never
//     blended), so the loop needs no per-entry bound test; each staged
//     record carries its list position for n_contrib.
//
// Per (pixel, entry), in this fixed fp32 order:
//   dx = u - px, dy = v - py
//   power = fma(dx, fma(-A/2, dx, -B*dy), (-C/2*dy)*dy)
//   skip if power > 0; alpha = min(0.99, o * exp(power)); skip if alpha < 1/255
//   T' = T (1 - alpha); stop before this entry if T' < 1e-4
//   w = alpha T; C_c = fma(rgb_c, w, C_c); T = T'
#include "raster_common.h"

namespace gs {

// The L1 loss fused at the end (L1 = true): each lane reads its pixel's
// target, writes dL/dimage = scale sign(I - I*) and the wave's sum of |I - I*|
// goes to partial[block] (0 for quarters outside the image); image may then
// be null.
template <bool L1>
__device__ __forceinline__ void raster_fwd_body(const float* __restrict__ rec, int64_t n,
                                                const uint32_t* __restrict__ ranges,
                                                const uint32_t* __restrict__ vals,
                                                const uint16_t* __restrict__ masks, int W, int H, int TX, int T,
                                                int row0, float bg0, float bg1, float bg2, float* __restrict__ image,
                                                float* __restrict__ T_final, int32_t* __restrict__ n_contrib,
                                                const float* __restrict__ target, float scale,
                                                float* __restrict__ dL, double* __restrict__ partial)
{
#pragma clang fp contract(off)
    // records at a stride of 48 bytes, and an extra slot of opacity 0 that
    // pads each row's list to the longest row's count (no pixel blends it)
    constexpr uint32_t SLOT_BYTES = 48, PAD_OFF = RW_BATCH * SLOT_BYTES;
    __shared__ float4 s_rec[3 * (RW_BATCH + 1)];
    __shared__ uint8_t s_mask[RW_BATCH];
    __shared__ __align__(16) uint16_t s_list[4 * RW_BATCH];  // record byte offsets, read 8 at a time
    const QuarterCtx t = quarter_ctx(W, H, TX, T, row0);
    if (t.empty) {
        if (L1 && t.lane == 0) partial[blockIdx.x] = 0.0;
        return;
    }
    // the target of this lane's pixel, requested now and used at the end
    float tg0 = 0.f, tg1 = 0.f, tg2 = 0.f;
    if (L1 && t.inside) {
        const int64_t HW = (int64_t)H * W;
        const int64_t o = (int64_t)t.view * 3 * HW + (int64_t)t.j * W + t.i;
        tg0 = target[o];
        tg1 = target[o + HW];
        tg2 = target[o + 2 * HW];
    }
    const uint2 rg = *(const uint2*)(ranges + 2 * (uint64_t)t.tile_lin);
    const float* rv = rec + (int64_t)t.view * n * GS_REC_FLOATS;
    float Tr = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    int32_t last = 0;
    bool done = !t.inside;
    if (t.lane == 0) {
        s_rec[3 * RW_BATCH] = make_float4(0.f, 0.f, 0.f, 0.f);
        s_rec[3 * RW_BATCH + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        s_rec[3 * RW_BATCH + 2] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const char* recb = (const char*)s_rec;
    // two-stage prefetch: records of batch k+1 and ids of batch k+2 are
    // requested while batch k is evaluated
    Entry cur, nxt, nx2;
    load_entry(cur, rg.x + t.lane < rg.y, rg.x + t.lane, vals, masks, t);
    gather_record(cur, rv);
    load_entry(nxt, rg.x + RW_BATCH + t.lane < rg.y, rg.x + RW_BATCH + t.lane, vals, masks, t);
    for (uint32_t base = rg.x; base < rg.y; base += RW_BATCH) {
        if (ballot(!done) == 0ull) break;
        stage_entry(cur, t.lane, (int32_t)(base - rg.x) + t.lane + 1, s_rec, s_mask);
        gather_record(nxt, rv);
        const uint32_t j2 = base + 2 * RW_BATCH + t.lane;
        load_entry(nx2, j2 < rg.y, j2, vals, masks, t);
        // per row, the staged entries of its sub-block in list order, as
        // record offsets; the rest of the row's list is the padding slot
        uint32_t cnt[4];
        {
            asm volatile("" ::: "memory");  // staging writes precede these reads (LDS is in order per wave)
            const uint32_t m4 = s_mask[t.lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = (m4 >> r) & 1u;
                const uint64_t m = ballot(keep);
                cnt[r] = (uint32_t)__popcll(m);
                if (keep) s_list[r * RW_BATCH + mask_rank(m)] = (uint16_t)(t.lane * SLOT_BYTES);
                if ((uint32_t)t.lane >= cnt[r]) s_list[r * RW_BATCH + t.lane] = (uint16_t)PAD_OFF;
            }
            asm volatile("" ::: "memory");  // list writes precede their reads
        }
        const uint32_t iters = max(max(cnt[0], cnt[1]), max(cnt[2], cnt[3]));
        const uint16_t* my_list = s_list + t.row * RW_BATCH;
        // groups of 8 entries: their record offsets in one 16-byte read
        for (uint32_t sb = 0; sb < iters; sb += 8) {
            const uint4 ids = *(const uint4*)(my_list + sb);
            const uint32_t idw[4] = {ids.x, ids.y, ids.z, ids.w};
#pragma unroll
            for (uint32_t i = 0; i < 8u; ++i) {
                if (sb + i >= iters) break;  // wave-uniform
                const uint32_t off = (idw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
                const float4 q0 = *(const float4*)(recb + off);
                const float4 q1 = *(const float4*)(recb + off + 16);
                const float2 q2 = *(const float2*)(recb + off + 32);
                // branch-free update: only lanes that blend change state (a
                // zero weight adds exactly 0)
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                const float alpha = fminf(ALPHA_MAX, q1.y * exp_fast(power));
                const float Tn = Tr * (1.f - alpha);
                const bool keep = !done && !(power > 0.f) && !(alpha < ALPHA_MIN);
                const bool stop = keep && Tn < T_MIN;
                const bool blend = keep && !stop;
                const float w = blend ? alpha * Tr : 0.f;
                C0 = __builtin_fmaf(q1.z, w, C0);
                C1 = __builtin_fmaf(q1.w, w, C1);
                C2 = __builtin_fmaf(q2.x, w, C2);
                Tr = blend ? Tn : Tr;
                last = blend ? __float_as_int(q2.y) : last;
                done = done || stop;
            }
            if (ballot(!done) == 0ull) break;
        }
        asm volatile("" ::: "memory");  // this batch's LDS reads precede the next staging
        cur = nxt;
        nxt.valid = nx2.valid;
        nxt.gid = nx2.gid;
        nxt.m4 = nx2.m4;
    }
    float ad = 0.f;  // |I - I*| summed over the channels
    if (t.inside) {
        const int64_t HW = (int64_t)H * W;
        const int64_t pix = (int64_t)t.j * W + t.i;
        const int64_t o = (int64_t)t.view * 3 * HW + pix;
        const float i0 = C0 + Tr * bg0, i1 = C1 + Tr * bg1, i2 = C2 + Tr * bg2;
        if (!L1 || image) {
            image[o] = i0;
            image[o + HW] = i1;
            image[o + 2 * HW] = i2;
        }
        T_final[(int64_t)t.view * HW + pix] = Tr;
        n_contrib[(int64_t)t.view * HW + pix] = last;
        if (L1) {
            const float d0 = i0 - tg0, d1 = i1 - tg1, d2 = i2 - tg2;
            dL[o] = d0 > 0.f ? scale : (d0 < 0.f ? -scale : 0.f);
            dL[o + HW] = d1 > 0.f ? scale : (d1 < 0.f ? -scale : 0.f);
            dL[o + 2 * HW] = d2 > 0.f ? scale : (d2 < 0.f ? -scale : 0.f);
            ad = (fabsf(d0) + fabsf(d1)) + fabsf(d2);
        }
    }
    if (L1) {
        double acc = (double)ad;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (t.lane == 0) partial[blockIdx.x] = acc;
    }
}

__global__ __launch_bounds__(RW_THREADS) void k_raster_fwd(const float* __restrict__ rec, int64_t n,
                                                           const uint32_t* __restrict__ ranges,
                                                           const uint32_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ masks, int W, int H, int TX,
                                                           int T, int row0, float bg0, float bg1, float bg2,
                                                           float* __restrict__ image, float* __restrict__ T_final,
                                                           int32_t* __restrict__ n_contrib)
{
    raster_fwd_body<false>(rec, n, ranges, vals, masks, W, H, TX, T, row0, bg0, bg1, bg2, image, T_final, n_contrib, nullptr, 0.f,
                           nullptr, nullptr);
}

__global__ __launch_bounds__(RW_THREADS) void k_raster_fwd_l1(const float* __restrict__ rec, int64_t n,
                                                              const uint32_t* __restrict__ ranges,
                                                              const uint32_t* __restrict__ vals,
                                                              const uint16_t* __restrict__ masks, int W, int H, int TX,
                                                              int T, int row0, float bg0, float bg1, float bg2,
                                                              float* __restrict__ image, float* __restrict__ T_final,
                                                              int32_t* __restrict__ n_contrib,
                                                              const float* __restrict__ target, float scale,
                                                              float* __restrict__ dL, double* __restrict__ partial)
{
    raster_fwd_body<true>(rec, n, ranges, vals, masks, W, H, TX, T, row0, bg0, bg1, bg2, image, T_final, n_contrib, target, scale,
                          dL, partial);
}

// loss += scale * sum of the per-quarter partial sums: each workgroup sums a
// contiguous slice, then one fp64 atomic per workgroup
__global__ __launch_bounds__(256) void k_loss_partials(const double* __restrict__ partial, int64_t count,
                                                       double scale, double* __restrict__ loss)
{
    __shared__ double s_w[4];
    const int64_t per = (count + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(count, b0 + per);
    double acc = 0.0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 256) acc += partial[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(loss, (((s_w[0] + s_w[1]) + s_w[2]) + s_w[3]) * scale);
}

}  // namespace gs

using namespace gs;

extern "C" {

size_t gs_rasterize_fwd_l1_workspace_bytes(int32_t n_views, int32_t width, int32_t height)
{
    if (n_views < 1 || n_views > GS_MAX_VIEWS || width <= 0 || height <= 0) return 0;
    const int64_t quarters = (int64_t)n_views * gs_tiles_x(width) * gs_tiles_y(height) * 4;
    return (size_t)quarters * sizeof(double);
}

gs_status gs_rasterize_fwd_l1(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                              const uint16_t* masks, const gs_camera* cams, int32_t n_views, int32_t row0,
                              int32_t rows, const float* bg, const float* target,
                              float scale, float* image, float* T_final, int32_t* n_contrib, float* dL_dimage,
                              double* loss, int32_t accumulate, void* ws, size_t ws_bytes, void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, cams, n_views, row0, rows, bg, a)) return GS_ERR_INVALID_ARGUMENT;
    if (!T_final || !n_contrib || !target || !dL_dimage || !loss || !ws) return GS_ERR_INVALID_ARGUMENT;
    if (ws_bytes < (size_t)a.n_blocks * sizeof(double)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    double* partial = (double*)ws;
    hipLaunchKernelGGL(k_raster_fwd_l1, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, s, rec, n, ranges, vals,
                       masks, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2], image, T_final,
                       n_contrib, target, scale, dL_dimage, partial);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    if (!accumulate && fill_u32((uint32_t*)loss, 2, 0u, s) != hipSuccess) return GS_ERR_HIP;
    const unsigned red_blocks = (unsigned)(a.n_blocks < 256 * 64 ? (a.n_blocks + 63) / 64 : 256);
    hipLaunchKernelGGL(k_loss_partials, dim3(red_blocks), dim3(256), 0, s, partial, a.n_blocks, (double)scale, loss);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_rasterize_fwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const uint16_t* masks, const gs_camera* cams, int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, float* image, float* T_final,
                           int32_t* n_contrib, void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, cams, n_views, row0, rows, bg, a)) return GS_ERR_INVALID_ARGUMENT;
    if (!image || !T_final || !n_contrib) return GS_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(k_raster_fwd, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, (hipStream_t)stream, rec, n,
                       ranges, vals, masks, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2],
                       image, T_final, n_contrib);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
