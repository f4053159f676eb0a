// gs_preprocess (Gaussian-wise projection + prefix sum of tile counts, or
// their total alone), gs_emit_intersections and gs_tile_ranges.
//
// Layout: parameters are [P][n] SoA, so a wave's 64 lanes read 64 consecutive
// floats of each row (one 256-byte line per row). Each lane writes its
// 48-byte record per view as three 16-byte stores.
#include <math.h>

#include <algorithm>

#include "internal.h"
#include "project.h"

namespace gs {

constexpr int PRE_THREADS = 256;

// Half-extent of the region where alpha = o exp(-d^T Q d / 2) reaches 1/255:
// the ellipse d^T Q d <= 2 ln(255 o), whose bounding half-widths are
// sqrt(tau a) and sqrt(tau c) (a, c the diagonal of Q^-1 = Sigma2). The
// threshold is widened (x1.002 + 0.01, +0.05 px) so that fp32 rounding of the
// per-pixel test can never fall outside it. Negative: no pixel can reach it.
__device__ __forceinline__ void alpha_extent(float o, float a, float c, float& ex, float& ey)
{
    const float t = 255.f * o;
    if (!(t > 1.f)) {
        ex = -1.f;
        ey = -1.f;
        return;
    }
    const float tau = 2.f * logf(t) * 1.002f + 0.01f;
    ex = sqrtf(tau * a) + 0.05f;
    ey = sqrtf(tau * c) + 0.05f;
}

// Whether a Gaussian with mean (x, y, z) and largest scale at most smax may
// be visible in the view: a superset of view_project's visible pairs, used
// only to skip the loads of Gaussians that cannot be. The camera transform
// and the projected mean are view_project's (same order); the 3-sigma radius
// is bounded through lambda_max(Sigma2) <= |J|_F^2 smax^2 + 0.3, with the
// Jacobian's guard-band clamp bounding x/z, y/z, and a margin of 1 % + 2 px.
__device__ __forceinline__ bool maybe_visible(float x, float y, float z, float smax, const DevCamera& cam, int TX,
                                              int TY)
{
#pragma clang fp contract(off)
    const float* W = cam.R;
    const float xc = ((W[0] * x + W[1] * y) + W[2] * z) + cam.t[0];
    const float yc = ((W[3] * x + W[4] * y) + W[5] * z) + cam.t[1];
    const float zc = ((W[6] * x + W[7] * y) + W[8] * z) + cam.t[2];
    if (!(zc > cam.near_plane && zc < cam.far_plane)) return false;
    const float jx = cam.fx / zc, jy = cam.fy / zc;
    const float lam = (jx * jx * (1.f + cam.limx * cam.limx) + jy * jy * (1.f + cam.limy * cam.limy)) * (smax * smax) + 0.3f;
    const float rb = 3.f * sqrtf(lam) * 1.01f + 2.f;
    const float u = (cam.fx * xc) / zc + cam.cx;
    const float v = (cam.fy * yc) / zc + cam.cy;
    return u + rb > 0.f && u - rb < 16.f * (float)TX && v + rb > 0.f && v - rb < 16.f * (float)TY;
}

// The 2D-gradient records of the wave's 64 Gaussians in view v are one
// contiguous block of 64 x 9 floats; the wave zeroes the whole block (dword
// stores, each instruction 256 contiguous bytes) when any of its lanes is
// visible in the view. Records of culled pairs in such a block are zeroed too
// (nothing reads them); blocks of waves with no visible lane are left alone.
__device__ __forceinline__ void zero_grad2d_block(float* __restrict__ g2z, int64_t n, int v, int64_t g0, bool any)
{
    if (!g2z || !any) return;  // wave-uniform
    const int64_t first = ((int64_t)v * n + g0) * GS_GRAD2D_ROWS;
    const int64_t count = (min(g0 + 64, n) - g0) * GS_GRAD2D_ROWS;
    const int64_t lane = (int64_t)(threadIdx.x & 63u);
#pragma unroll
    for (int k = 0; k < GS_GRAD2D_ROWS; ++k)
        if (lane + 64 * k < count) g2z[first + lane + 64 * k] = 0.f;
}

// One thread per Gaussian. The means and log-scales are loaded first; a
// Gaussian that no view can see (maybe_visible) writes its zero counts and
// empty rectangles without loading the rest, so that the waves of a scene
// stored in a spatial order that lie outside every view read 24 of 236 bytes.
// The others load their remaining rows together, then every view is pure
// arithmetic plus the record stores. The per-(view, Gaussian) tile counts go
// to `counts` when it is given; with `wave_sums`, each wave's sum of them goes
// to wave_sums[g / 64] (for the total alone, without the offsets), and the
// first thread zeroes *total, which k_sum_counts then adds to.
template <int DEG>
__global__ __launch_bounds__(PRE_THREADS) void k_preprocess(const float* __restrict__ P, int64_t n,
                                                            const DevCameras cams, const ShConsts K,
                                                            float* __restrict__ rec, uint16_t* __restrict__ rect,
                                                            float* __restrict__ depth, float* __restrict__ g2zero,
                                                            uint32_t* __restrict__ counts,
                                                            uint32_t* __restrict__ wave_sums,
                                                            uint64_t* __restrict__ total)
{
    if (wave_sums && blockIdx.x == 0 && threadIdx.x == 0) *total = 0;
    constexpr int NB = (DEG + 1) * (DEG + 1);
    const int64_t g = (int64_t)blockIdx.x * PRE_THREADS + threadIdx.x;
    const int64_t g0 = g & ~(int64_t)63;  // the wave's first Gaussian
    if (g0 >= n) return;                   // whole waves past the end
    const bool here = g < n;
    float raw[11];
#pragma unroll
    for (int r = 0; r < 6; ++r) raw[r] = here ? P[(int64_t)r * n + g] : 0.f;
    bool maybe = false;
    if (here) {
        const float smax = __expf(fmaxf(raw[3], fmaxf(raw[4], raw[5]))) * 1.001f;
        for (int v = 0; v < cams.n_views; ++v)
            maybe = maybe || maybe_visible(raw[0], raw[1], raw[2], smax, cams.c[v], cams.tiles_x, cams.tiles_y);
    }
    if (!maybe) {
        // no view can see it: zero counts, empty rectangles, nothing loaded
        if (here)
            for (int v = 0; v < cams.n_views; ++v) {
                const int64_t idx = (int64_t)v * n + g;
                if (counts) counts[idx] = 0u;
                *(uint2*)(rect + 4 * idx) = make_uint2(0u, 0u);
            }
    }
    uint32_t vis_bits = 0u;  // bit v: visible in view v
    uint32_t my_count = 0u;  // tile count summed over the views
    if (maybe) {
#pragma unroll
        for (int r = 6; r < 11; ++r) raw[r] = P[(int64_t)r * n + g];
        float sh[3 * NB];
#pragma unroll
        for (int k = 0; k < 3 * NB; ++k) sh[k] = P[(int64_t)(11 + k) * n + g];
        const float x = raw[0], y = raw[1], z = raw[2];
        GaussLocal L;
        gauss_local(raw[3], raw[4], raw[5], raw[6], raw[7], raw[8], raw[9], raw[10], L);
        for (int v = 0; v < cams.n_views; ++v) {
            const DevCamera& cam = cams.c[v];
            ViewProj p;
            view_project(x, y, z, L, cam, cams.tiles_x, cams.tiles_y, p);
            const int64_t idx = (int64_t)v * n + g;
            if (!p.visible) {
                if (counts) counts[idx] = 0u;
                *(uint2*)(rect + 4 * idx) = make_uint2(0u, 0u);
                continue;
            }
            vis_bits |= 1u << v;
            float d[3], dist;
            view_dir(x, y, z, cam, d, dist);
            float Y[16];
            sh_eval_basis(K, DEG, d, Y);
            bool cl;
            const float r = sh_channel_reg<NB>(sh, 0, Y, cl);
            const float gg = sh_channel_reg<NB>(sh, 1, Y, cl);
            const float b = sh_channel_reg<NB>(sh, 2, Y, cl);
            float ex, ey;
            alpha_extent(L.o, p.a, p.c, ex, ey);
            float4* out = (float4*)(rec + idx * GS_REC_FLOATS);
            out[0] = make_float4(p.u, p.v, p.A, p.B);
            out[1] = make_float4(p.C, L.o, r, gg);
            out[2] = make_float4(b, ex, ey, p.zc);
            if (depth) depth[idx] = p.zc;
            *(uint2*)(rect + 4 * idx) = make_uint2((uint32_t)p.x0 | ((uint32_t)p.y0 << 16),
                                                   (uint32_t)p.x1 | ((uint32_t)p.y1 << 16));
            const uint32_t cnt = (uint32_t)((p.x1 - p.x0) * (p.y1 - p.y0));
            if (counts) counts[idx] = cnt;
            my_count += cnt;
        }
    }
    if (wave_sums) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) my_count += __shfl_xor(my_count, off);
        if ((threadIdx.x & 63u) == 0u) wave_sums[g0 >> 6] = my_count;
    }
    if (g2zero)
        for (int v = 0; v < cams.n_views; ++v) zero_grad2d_block(g2zero, n, v, g0, ballot((vis_bits >> v) & 1u) != 0ull);
}

// *total (zeroed by k_preprocess) += the sum of `count` wave sums: each
// workgroup sums a contiguous slice and adds it with one 64-bit integer
// atomic (exact in any order).
constexpr int SUM_THREADS = 256;
__global__ __launch_bounds__(SUM_THREADS) void k_sum_counts(const uint32_t* __restrict__ s, int64_t count,
                                                            uint64_t* __restrict__ total)
{
    __shared__ uint64_t w[SUM_THREADS / 64];
    const int64_t per = (count + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(count, b0 + per);
    uint64_t acc = 0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += SUM_THREADS) acc += s[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63u) == 0u) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t t = (w[0] + w[1]) + (w[2] + w[3]);
        if (t) atomicAdd((unsigned long long*)total, (unsigned long long)t);
    }
}

// One thread per (view, Gaussian): its tiles in row-major order, at its offset.
__global__ __launch_bounds__(256) void k_emit(const float* __restrict__ rec, const uint16_t* __restrict__ rect,
                                              const uint32_t* __restrict__ offsets, int64_t n, int64_t total_entries,
                                              int32_t tiles_x, int64_t tiles_per_view, uint64_t* __restrict__ keys,
                                              uint32_t* __restrict__ vals, uint64_t capacity,
                                              int32_t* __restrict__ overflow)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total_entries) return;
    const uint2 rr = *(const uint2*)(rect + 4 * idx);
    const uint32_t x0 = rr.x & 0xffffu, y0 = rr.x >> 16, x1 = rr.y & 0xffffu, y1 = rr.y >> 16;
    if (x1 <= x0 || y1 <= y0) return;
    const int64_t v = idx / n, g = idx - v * n;
    const uint32_t zb = __float_as_uint(rec[idx * GS_REC_FLOATS + GS_REC_DEPTH]);
    uint64_t k = offsets[idx];
    const uint64_t tbase = (uint64_t)v * (uint64_t)tiles_per_view;
    bool over = false;
    for (uint32_t ty = y0; ty < y1; ++ty)
        for (uint32_t tx = x0; tx < x1; ++tx, ++k) {
            if (k >= capacity) {
                over = true;
                continue;
            }
            keys[k] = ((tbase + (uint64_t)ty * tiles_x + tx) << 32) | zb;
            vals[k] = (uint32_t)g;
        }
    if (over) *overflow = 1;
}

__global__ __launch_bounds__(256) void k_ranges(const uint64_t* __restrict__ keys, uint64_t n_keys,
                                                uint64_t n_tiles_total, uint32_t* __restrict__ ranges)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_keys) return;
    const uint32_t t = (uint32_t)(keys[i] >> 32);
    if (t >= n_tiles_total) return;  // not a key of this tile grid
    if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * (uint64_t)t] = (uint32_t)i;
    if (i + 1 == n_keys || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * (uint64_t)t + 1] = (uint32_t)(i + 1);
}

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_preprocess(const float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                        int32_t n_views, float* rec, uint16_t* rect, float* depth, float* grad2d, uint32_t* offsets,
                        uint64_t* total, void* ws, size_t ws_bytes, void* stream)
{
    if (n < 0 || sh_degree < 0 || sh_degree > 3) return GS_ERR_INVALID_ARGUMENT;
    if (!total || !ws) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !rec || !rect)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    DevCameras dc;
    if (!make_dev_cameras(cams, n_views, dc)) return GS_ERR_INVALID_ARGUMENT;
    const uint64_t entries = (uint64_t)n * (uint64_t)n_views;
    const int64_t waves = (n + 63) / 64;
    if (ws_bytes < (offsets ? scan_workspace_bytes(entries) : (size_t)waves * 4)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    uint32_t* wave_sums = offsets ? nullptr : (uint32_t*)ws;
    if (n > 0) {
        const dim3 grid(grid_for((uint64_t)n, PRE_THREADS)), block(PRE_THREADS);
        const ShConsts K = sh_constants();
        switch (sh_degree) {
            case 0: hipLaunchKernelGGL(k_preprocess<0>, grid, block, 0, s, params, n, dc, K, rec, rect, depth, grad2d, offsets, wave_sums, total); break;
            case 1: hipLaunchKernelGGL(k_preprocess<1>, grid, block, 0, s, params, n, dc, K, rec, rect, depth, grad2d, offsets, wave_sums, total); break;
            case 2: hipLaunchKernelGGL(k_preprocess<2>, grid, block, 0, s, params, n, dc, K, rec, rect, depth, grad2d, offsets, wave_sums, total); break;
            default: hipLaunchKernelGGL(k_preprocess<3>, grid, block, 0, s, params, n, dc, K, rec, rect, depth, grad2d, offsets, wave_sums, total); break;
        }
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    }
    if (offsets) {
        // counts were written into `offsets`; scan them in place
        if (scan_u32(offsets, offsets, entries, total, ws, s) != hipSuccess) return GS_ERR_HIP;
        return GS_OK;
    }
    if (n == 0) return fill_u32((uint32_t*)total, 2, 0u, s) == hipSuccess ? GS_OK : GS_ERR_HIP;
    // a workgroup per 2048 wave sums, at most 1024 workgroups
    const unsigned sum_blocks = (unsigned)std::min<int64_t>(1024, (waves + 2047) / 2048);
    hipLaunchKernelGGL(k_sum_counts, dim3(sum_blocks), dim3(SUM_THREADS), 0, s, wave_sums, waves, total);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_emit_intersections(const float* rec, const uint16_t* rect, const uint32_t* offsets, int64_t n,
                                int32_t n_views, int32_t width, int32_t height, uint64_t* keys, uint32_t* vals,
                                uint64_t capacity, int32_t* overflow, void* stream)
{
    if (n < 0 || n_views < 1 || n_views > GS_MAX_VIEWS || width <= 0 || height <= 0)
        return GS_ERR_INVALID_ARGUMENT;
    if (!offsets || !overflow) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!rec || !rect)) return GS_ERR_INVALID_ARGUMENT;
    if (capacity > 0 && (!keys || !vals)) return GS_ERR_INVALID_ARGUMENT;
    const int64_t tx = gs_tiles_x(width), tpv = tx * gs_tiles_y(height);
    if (tpv * n_views >= ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    const int64_t entries = n * n_views;
    if (fill_u32((uint32_t*)overflow, 1, 0u, (hipStream_t)stream) != hipSuccess) return GS_ERR_HIP;
    if (entries == 0) return GS_OK;
    hipLaunchKernelGGL(k_emit, dim3(grid_for((uint64_t)entries, 256)), dim3(256), 0, (hipStream_t)stream, rec,
                       rect, offsets, n, entries, (int32_t)tx, tpv, keys, vals, capacity, overflow);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_tile_ranges(const uint64_t* keys, uint64_t n_keys, int64_t n_tiles_total, uint32_t* ranges,
                         void* stream)
{
    if (n_tiles_total < 0 || !ranges || (n_keys > 0 && !keys)) return GS_ERR_INVALID_ARGUMENT;
    if (n_keys >= ((uint64_t)1 << 32)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (fill_u32(ranges, 2 * (uint64_t)n_tiles_total, 0u, s) != hipSuccess) return GS_ERR_HIP;
    if (n_keys > 0) {
        hipLaunchKernelGGL(k_ranges, dim3(grid_for(n_keys, 256)), dim3(256), 0, s, keys, n_keys,
                           (uint64_t)n_tiles_total, ranges);
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    }
    return GS_OK;
}

}  // extern "C"
