// gs_rasterize_fwd / gs_rasterize_bwd: per-tile alpha compositing over the
// sorted intersection lists and its reverse-order backward pass (forward and
// backward rasterization of the ByteSplat abstract; 16x16 pixel blocks of "On
// Scaling Up 3D Gaussian Splatting Training", answer (1)).
//
// Work unit: one wavefront (one 64-thread workgroup) per 8x8 quarter of a
// 16x16 tile, one lane per pixel. Waves are independent, so each stops as soon
// as its own 64 pixels are saturated. The tile's list is walked in batches of
// 64 entries: every lane fetches one entry's record (a 48-byte gather), tests
// whether the region where the entry's alpha can reach 1/255 touches the
// wave's 8x8 block, and the survivors are compacted into LDS with a ballot
// (order kept). The pixel loop then reads each survivor once as an LDS
// broadcast. An entry culled this way has alpha < 1/255 at every pixel of the
// block, so it would have been skipped anyway: the result is unchanged.
//
// Per (pixel, entry), in this fixed fp32 order:
//   dx = u - px, dy = v - py
//   power = fma(dx, fma(-A/2, dx, -B*dy), (-C/2*dy)*dy)
//   skip if power > 0; alpha = min(0.99, o * exp(power)); skip if alpha < 1/255
//   T' = T (1 - alpha); stop before this entry if T' < 1e-4
//   w = alpha T; C_c = fma(rgb_c, w, C_c); T = T'
#include "internal.h"

namespace gs {

constexpr float ALPHA_MIN = 1.0f / 255.0f;
constexpr float ALPHA_MAX = 0.99f;
constexpr float T_MIN = 1e-4f;
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

struct TileWave {
    uint32_t view, tile_lin;  // tile_lin = view * tiles_per_view + tile
    int i, j;                 // this lane's pixel
    bool inside;
    float px, py;
    float bx0, bx1, by0, by1;  // box of the wave's pixel centres
    bool empty;                // the wave's block lies outside the image
};

__device__ __forceinline__ TileWave tile_wave(uint32_t nblocks, int W, int H, int TX, int T)
{
    TileWave t;
    const uint32_t lb = xcd_contiguous(blockIdx.x, nblocks);
    const uint32_t quad = lb & 3u;
    t.tile_lin = lb >> 2;
    t.view = t.tile_lin / (uint32_t)T;
    const uint32_t tile = t.tile_lin - t.view * (uint32_t)T;
    const uint32_t ty = tile / (uint32_t)TX, tx = tile - ty * (uint32_t)TX;
    const int x0 = (int)tx * 16 + (int)(quad & 1u) * 8, y0 = (int)ty * 16 + (int)(quad >> 1) * 8;
    const int lane = (int)threadIdx.x;
    t.i = x0 + (lane & 7);
    t.j = y0 + (lane >> 3);
    t.inside = t.i < W && t.j < H;
    t.px = (float)t.i + 0.5f;
    t.py = (float)t.j + 0.5f;
    t.empty = x0 >= W || y0 >= H;
    t.bx0 = (float)x0 + 0.5f;
    t.by0 = (float)y0 + 0.5f;
    t.bx1 = (float)min(x0 + 8, W) - 0.5f;
    t.by1 = (float)min(y0 + 8, H) - 0.5f;
    return t;
}

// Fetch list entry `jj` (this lane), test it against the wave box and stage
// the survivors in LDS in list order. Returns the number staged.
// Staged layout, 3 x float4 per entry:
//   (u, v, -A/2, -B) (-C/2, o, r, g) (b, position, gid, -)
__device__ __forceinline__ uint32_t stage_batch(bool valid, uint32_t jj, uint32_t pos, const float* __restrict__ rv,
                                                const uint32_t* __restrict__ vals, const TileWave& t,
                                                float4* __restrict__ s)
{
    bool keep = false;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a, c = a;
    uint32_t gid = 0;
    if (valid) {
        gid = vals[jj];
        const float4* rp = (const float4*)(rv + (int64_t)gid * GS_REC_FLOATS);
        a = rp[0];  // u v A B
        b = rp[1];  // C o r g
        c = rp[2];  // b ex ey z
        keep = (a.x + c.y >= t.bx0) && (a.x - c.y <= t.bx1) && (a.y + c.z >= t.by0) && (a.y - c.z <= t.by1);
    }
    const uint64_t m = ballot(keep);
    if (keep) {
        const uint32_t slot = mask_rank(m);
        s[3 * slot + 0] = make_float4(a.x, a.y, -0.5f * a.z, -a.w);
        s[3 * slot + 1] = make_float4(-0.5f * b.x, b.y, b.z, b.w);
        s[3 * slot + 2] = make_float4(c.x, __uint_as_float(pos), __uint_as_float(gid), 0.f);
    }
    return (uint32_t)__popcll(m);
}

__device__ __forceinline__ float entry_power(const float4& q0, const float4& q1, float px, float py, float& dx,
                                             float& dy)
{
#pragma clang fp contract(off)
    dx = q0.x - px;
    dy = q0.y - py;
    return __builtin_fmaf(dx, __builtin_fmaf(q0.z, dx, q0.w * dy), (q1.x * dy) * dy);
}

__global__ __launch_bounds__(64) void k_raster_fwd(const float* __restrict__ rec, int64_t n,
                                                   const uint32_t* __restrict__ ranges,
                                                   const uint32_t* __restrict__ vals, int W, int H, int TX, int T,
                                                   float bg0, float bg1, float bg2, float* __restrict__ image,
                                                   float* __restrict__ T_final, int32_t* __restrict__ n_contrib)
{
#pragma clang fp contract(off)
    __shared__ float4 s[3 * 64];
    const TileWave t = tile_wave(gridDim.x, W, H, TX, T);
    if (t.empty) return;
    const uint2 rg = *(const uint2*)(ranges + 2 * (uint64_t)t.tile_lin);
    const float* rv = rec + (int64_t)t.view * n * GS_REC_FLOATS;
    float Tr = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    int32_t last = 0;
    bool done = !t.inside;
    for (uint32_t base = rg.x; base < rg.y; base += 64) {
        if (ballot(!done) == 0ull) break;
        const uint32_t jj = base + threadIdx.x;
        const uint32_t cnt = stage_batch(jj < rg.y, jj, jj - rg.x + 1u, rv, vals, t, s);
        __syncthreads();
        for (uint32_t e = 0; e < cnt; ++e) {
            const float4 q0 = s[3 * e], q1 = s[3 * e + 1], q2 = s[3 * e + 2];
            if (!done) {
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                if (!(power > 0.f)) {
                    const float alpha = fminf(ALPHA_MAX, q1.y * exp_fast(power));
                    if (!(alpha < ALPHA_MIN)) {
                        const float Tn = Tr * (1.f - alpha);
                        if (Tn < T_MIN) {
                            done = true;
                        } else {
                            const float w = alpha * Tr;
                            C0 = __builtin_fmaf(q1.z, w, C0);
                            C1 = __builtin_fmaf(q1.w, w, C1);
                            C2 = __builtin_fmaf(q2.x, w, C2);
                            Tr = Tn;
                            last = (int32_t)__float_as_uint(q2.y);
                        }
                    }
                }
            }
            if (ballot(!done) == 0ull) break;
        }
        __syncthreads();
    }
    if (t.inside) {
        const int64_t HW = (int64_t)H * W;
        const int64_t pix = (int64_t)t.j * W + t.i;
        float* img = image + (int64_t)t.view * 3 * HW + pix;
        img[0] = C0 + Tr * bg0;
        img[HW] = C1 + Tr * bg1;
        img[2 * HW] = C2 + Tr * bg2;
        T_final[(int64_t)t.view * HW + pix] = Tr;
        n_contrib[(int64_t)t.view * HW + pix] = last;
    }
}

__global__ __launch_bounds__(64) void k_raster_bwd(const float* __restrict__ rec, int64_t n,
                                                   const uint32_t* __restrict__ ranges,
                                                   const uint32_t* __restrict__ vals, int W, int H, int TX, int T,
                                                   float bg0, float bg1, float bg2,
                                                   const float* __restrict__ T_final,
                                                   const int32_t* __restrict__ n_contrib,
                                                   const float* __restrict__ dL_dimage, float* __restrict__ grad2d)
{
#pragma clang fp contract(off)
    __shared__ float4 s[3 * 64];
    const TileWave t = tile_wave(gridDim.x, W, H, TX, T);
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
    if (g0 == 0.f && g1 == 0.f && g2 == 0.f) my_last = 0;  // this pixel adds nothing
    const uint2 rg = *(const uint2*)(ranges + 2 * (uint64_t)t.tile_lin);
    // never walk past the tile's list, whatever n_contrib holds
    const int32_t wave_last = min(wave_max_int(my_last), (int32_t)(rg.y - rg.x));
    if (wave_last <= 0) return;
    const float* rv = rec + (int64_t)t.view * n * GS_REC_FLOATS;
    float* g2d = grad2d + (int64_t)t.view * GS_GRAD2D_ROWS * n;
    // colour behind the current entry, normalised by the transmittance in
    // front of it; starts as the background behind the last blended entry
    float acc0 = bg0, acc1 = bg1, acc2 = bg2;
    for (int32_t hi = wave_last; hi >= 1; hi -= 64) {
        const int32_t p = hi - (int32_t)threadIdx.x;  // list position (1-based), descending over lanes
        const uint32_t cnt = stage_batch(p >= 1, rg.x + (uint32_t)(p - 1), (uint32_t)p, rv, vals, t, s);
        __syncthreads();
        for (uint32_t e = 0; e < cnt; ++e) {
            const float4 q0 = s[3 * e], q1 = s[3 * e + 1], q2 = s[3 * e + 2];
            const int32_t pos = (int32_t)__float_as_uint(q2.y);
            float gu = 0.f, gv = 0.f, gA = 0.f, gB = 0.f, gC = 0.f, go = 0.f, gr = 0.f, gg = 0.f, gb = 0.f;
            bool contrib = false;
            if (pos <= my_last) {
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                if (!(power > 0.f)) {
                    const float G = exp_fast(power);
                    const float oG = q1.y * G;
                    const float alpha = fminf(ALPHA_MAX, oG);
                    if (!(alpha < ALPHA_MIN)) {
                        contrib = true;
                        Tr = Tr / (1.f - alpha);  // transmittance in front of this entry
                        const float w = alpha * Tr;
                        gr = w * g0;
                        gg = w * g1;
                        gb = w * g2;
                        const float dLda = Tr * (((q1.z - acc0) * g0 + (q1.w - acc1) * g1) + (q2.x - acc2) * g2);
                        const float om = 1.f - alpha;
                        acc0 = alpha * q1.z + om * acc0;
                        acc1 = alpha * q1.w + om * acc1;
                        acc2 = alpha * q2.x + om * acc2;
                        if (!(oG > ALPHA_MAX)) {
                            go = dLda * G;
                            const float dp = dLda * oG;  // dL/dpower
                            gu = dp * (2.f * q0.z * dx + q0.w * dy);
                            gv = dp * (q0.w * dx + 2.f * q1.x * dy);
                            gA = -0.5f * dp * (dx * dx);
                            gB = -dp * (dx * dy);
                            gC = -0.5f * dp * (dy * dy);
                        }
                    }
                }
            }
            if (ballot(contrib) != 0ull) {
                const float r0 = wave_sum(gu), r1 = wave_sum(gv), r2 = wave_sum(gA), r3 = wave_sum(gB),
                            r4 = wave_sum(gC), r5 = wave_sum(go), r6 = wave_sum(gr), r7 = wave_sum(gg),
                            r8 = wave_sum(gb);
                const uint32_t lane = threadIdx.x;
                float val = r0;
                val = lane == 1 ? r1 : val;
                val = lane == 2 ? r2 : val;
                val = lane == 3 ? r3 : val;
                val = lane == 4 ? r4 : val;
                val = lane == 5 ? r5 : val;
                val = lane == 6 ? r6 : val;
                val = lane == 7 ? r7 : val;
                val = lane == 8 ? r8 : val;
                if (lane < GS_GRAD2D_ROWS) {
                    const uint32_t gid = __float_as_uint(q2.z);
                    atomicAdd(g2d + (int64_t)lane * n + gid, val);
                }
            }
        }
        __syncthreads();
    }
}

struct RasterArgs {
    DevCameras dc;
    int64_t n_blocks;
};

static bool raster_args(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                        const gs_camera* cams, int32_t n_views, const float* bg, RasterArgs& a)
{
    if (n < 0 || !ranges || !bg) return false;
    if (n > 0 && (!rec || !vals)) return false;
    if (!make_dev_cameras(cams, n_views, a.dc)) return false;
    a.n_blocks = (int64_t)n_views * a.dc.tiles_per_view * 4;
    return a.n_blocks < ((int64_t)1 << 31);
}

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_rasterize_fwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const gs_camera* cams, int32_t n_views, const float* bg, float* image, float* T_final,
                           int32_t* n_contrib, void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, cams, n_views, bg, a)) return GS_ERR_INVALID_ARGUMENT;
    if (!image || !T_final || !n_contrib) return GS_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(k_raster_fwd, dim3((unsigned)a.n_blocks), dim3(64), 0, (hipStream_t)stream, rec, n, ranges,
                       vals, a.dc.width, a.dc.height, a.dc.tiles_x, a.dc.tiles_per_view, bg[0], bg[1], bg[2], image,
                       T_final, n_contrib);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_rasterize_bwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const gs_camera* cams, int32_t n_views, const float* bg, const float* T_final,
                           const int32_t* n_contrib, const float* dL_dimage, float* grad2d, int32_t accumulate,
                           void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, cams, n_views, bg, a)) return GS_ERR_INVALID_ARGUMENT;
    if (!T_final || !n_contrib || !dL_dimage || (n > 0 && !grad2d)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate && n > 0) {
        if (fill_u32((uint32_t*)grad2d, (uint64_t)n_views * GS_GRAD2D_ROWS * (uint64_t)n, 0u, s) != hipSuccess)
            return GS_ERR_HIP;
    }
    hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)a.n_blocks), dim3(64), 0, s, rec, n, ranges, vals, a.dc.width,
                       a.dc.height, a.dc.tiles_x, a.dc.tiles_per_view, bg[0], bg[1], bg[2], T_final, n_contrib,
                       dL_dimage, grad2d);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
