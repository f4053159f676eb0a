// gs_rasterize_fwd_bwd_l1: forward rasterization, L1 loss and backward
// rasterization of the ByteSplat abstract in one pass per 8x8 quarter. The L1
// gradient of a pixel depends on that pixel alone (sign(I - I*)), so the
// wavefront that blended a quarter's pixels can walk its list back at once
// with T_final, n_contrib and dL/dimage still in registers: they need not go
// through device memory, and the list is walked by the same wave twice
// without a second launch. The forward walk (raster_fwd.h) and the backward
// walk (raster_bwd.h) share one LDS allocation, used by one after the other.
#include <mutex>

#include "raster_bwd.h"
#include "raster_fwd.h"

namespace gs {

constexpr size_t FUSED_LDS_BYTES = sizeof(FwdLds) > sizeof(BwdLds) ? sizeof(FwdLds) : sizeof(BwdLds);

// The order in which the pass takes the (view, tile)s: by list length, longest
// first, in ORDER_CLASSES classes, tile order within a class. A quarter's time
// grows with its tile's list, and in tile order the quarters of long lists
// that start late finish long after the rest. A counting sort over segments of
// ORDER_SEG tiles: k_order_count counts each segment's classes, k_order_place
// adds the counts of the classes before and of the segments before, and ranks
// the segment's tiles by ballots (tile = segment base + 256 r + 64 wave + lane,
// so rank order is tile order).
constexpr int ORDER_CLASSES = 8;
constexpr int ORDER_THREADS = 256;
constexpr int ORDER_R = 4;  // tiles per thread
constexpr int ORDER_SEG = ORDER_THREADS * ORDER_R;

__device__ __forceinline__ int order_class(uint32_t len)
{
    // > 4096, > 2048, > 1024, > 512, > 256, > 128, > 64, the rest
    int c = 0;
#pragma unroll
    for (int k = 12; k >= 6; --k) c += len <= (1u << k) ? 1 : 0;
    return c;
}

// the classes of this thread's ORDER_R tiles (ORDER_CLASSES past the end)
__device__ __forceinline__ void segment_classes(const uint32_t* __restrict__ ranges, int64_t n_tiles,
                                                int (&c)[ORDER_R])
{
    const int64_t base = (int64_t)blockIdx.x * ORDER_SEG + threadIdx.x;
    uint2 rg[ORDER_R];
#pragma unroll
    for (int r = 0; r < ORDER_R; ++r) {
        const int64_t t = base + r * ORDER_THREADS;
        rg[r] = t < n_tiles ? *(const uint2*)(ranges + 2 * t) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < ORDER_R; ++r)
        c[r] = base + r * ORDER_THREADS < n_tiles ? order_class(rg[r].y - rg[r].x) : ORDER_CLASSES;
}

// table[segment][class]: the segment's tiles of each class
__global__ __launch_bounds__(ORDER_THREADS) void k_order_count(const uint32_t* __restrict__ ranges, int64_t n_tiles,
                                                              uint32_t* __restrict__ table)
{
    __shared__ uint32_t cnt[ORDER_CLASSES];
    if (threadIdx.x < ORDER_CLASSES) cnt[threadIdx.x] = 0u;
    int c[ORDER_R];
    segment_classes(ranges, n_tiles, c);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ORDER_CLASSES; ++k) {
        uint32_t m = 0u;
#pragma unroll
        for (int r = 0; r < ORDER_R; ++r) m += (uint32_t)__popcll(ballot(c[r] == k));
        if ((threadIdx.x & 63u) == 0u && m) atomicAdd(&cnt[k], m);
    }
    __syncthreads();
    if (threadIdx.x < ORDER_CLASSES) table[(int64_t)blockIdx.x * ORDER_CLASSES + threadIdx.x] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(ORDER_THREADS) void k_order_place(const uint32_t* __restrict__ ranges, int64_t n_tiles,
                                                              const uint32_t* __restrict__ table, uint32_t n_seg,
                                                              uint32_t* __restrict__ order)
{
    constexpr int W = ORDER_THREADS / 64;
    __shared__ uint32_t tot[ORDER_CLASSES], before[ORDER_CLASSES];
    __shared__ uint32_t cnt[ORDER_R][W][ORDER_CLASSES];  // then: first slot of each (r, wave, class)
    if (threadIdx.x < ORDER_CLASSES) tot[threadIdx.x] = before[threadIdx.x] = 0u;
    int c[ORDER_R];
    segment_classes(ranges, n_tiles, c);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_seg * ORDER_CLASSES; i += ORDER_THREADS) {
        const uint32_t v = table[i], k = i % ORDER_CLASSES;
        if (v) {
            atomicAdd(&tot[k], v);
            if (i / ORDER_CLASSES < blockIdx.x) atomicAdd(&before[k], v);
        }
    }
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint32_t rank[ORDER_R];
#pragma unroll
    for (int r = 0; r < ORDER_R; ++r) {
        rank[r] = 0u;
#pragma unroll
        for (int k = 0; k < ORDER_CLASSES; ++k) {
            const uint64_t m = ballot(c[r] == k);
            if (c[r] == k) rank[r] = mask_rank(m);
            if (lane == 0u) cnt[r][w][k] = (uint32_t)__popcll(m);
        }
    }
    __syncthreads();
    if (threadIdx.x < ORDER_CLASSES) {
        const int k = (int)threadIdx.x;
        uint32_t run = before[k];
        for (int j = 0; j < k; ++j) run += tot[j];
        for (int r = 0; r < ORDER_R; ++r)
            for (int v = 0; v < W; ++v) {
                const uint32_t x = cnt[r][v][k];
                cnt[r][v][k] = run;
                run += x;
            }
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * ORDER_SEG + threadIdx.x;
#pragma unroll
    for (int r = 0; r < ORDER_R; ++r)
        if (c[r] < ORDER_CLASSES) order[cnt[r][w][c[r]] + rank[r]] = (uint32_t)(base + r * ORDER_THREADS);
}

// image, T_final, n_contrib and dL may each be null (not written).
__global__ __launch_bounds__(RW_THREADS) void k_raster_fwd_bwd_l1(
    const float* __restrict__ rec, int64_t n, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ vals,
    const uint16_t* __restrict__ masks, uint32_t cap, int W, int H, int TX, int T, int row0, float bg0, float bg1,
    float bg2,
    const float* __restrict__ target, float scale, float* __restrict__ image, float* __restrict__ T_final,
    int32_t* __restrict__ n_contrib, float* __restrict__ dL, double* __restrict__ partial,
    float* __restrict__ grad2d, const uint32_t* __restrict__ order)
{
#pragma clang fp contract(off)
    __shared__ __align__(16) unsigned char lds[FUSED_LDS_BYTES];
    if (blockIdx.x == 0 && threadIdx.x == 0) *loss_counter(partial, gridDim.x) = 0u;
    const QuarterCtx t = quarter_ctx(W, H, TX, T, row0, order);
    if (t.empty) {
        if (t.lane == 0) partial[blockIdx.x] = 0.0;
        return;
    }
    const int64_t HW = (int64_t)H * W;
    const int64_t pix = (int64_t)t.j * W + t.i;
    const int64_t o = (int64_t)t.view * 3 * HW + pix;
    float tg0 = 0.f, tg1 = 0.f, tg2 = 0.f;
    if (t.inside) {  // read once per step: streamed past the caches
        tg0 = __builtin_nontemporal_load(target + o);
        tg1 = __builtin_nontemporal_load(target + o + HW);
        tg2 = __builtin_nontemporal_load(target + o + 2 * HW);
    }
    const FwdPixel P = raster_fwd_walk(*reinterpret_cast<FwdLds*>(lds), t, rec, n, ranges, vals, masks, cap);
    float g0 = 0.f, g1 = 0.f, g2 = 0.f, ad = 0.f;
    int32_t last = 0;
    if (t.inside) {
        const float i0 = P.C0 + P.Tr * bg0, i1 = P.C1 + P.Tr * bg1, i2 = P.C2 + P.Tr * bg2;
        const float d0 = i0 - tg0, d1 = i1 - tg1, d2 = i2 - tg2;
        g0 = l1_grad(d0, scale);
        g1 = l1_grad(d1, scale);
        g2 = l1_grad(d2, scale);
        ad = (fabsf(d0) + fabsf(d1)) + fabsf(d2);
        last = P.last;
        if (image) {
            image[o] = i0;
            image[o + HW] = i1;
            image[o + 2 * HW] = i2;
        }
        if (T_final) T_final[(int64_t)t.view * HW + pix] = P.Tr;
        if (n_contrib) n_contrib[(int64_t)t.view * HW + pix] = P.last;
        if (dL) {
            dL[o] = g0;
            dL[o + HW] = g1;
            dL[o + 2 * HW] = g2;
        }
    }
    loss_partial(ad, t.lane, partial);
    asm volatile("" ::: "memory");  // the forward's LDS reads precede the backward's writes (in order per wave)
    raster_bwd_walk(*reinterpret_cast<BwdLds*>(lds), t, last, P.Tr, g0, g1, g2, bg0, bg1, bg2, rec, n, ranges, vals,
                    masks, cap, grad2d);
}

}  // namespace gs

using namespace gs;

extern "C" {

// per quarter a loss partial, then the loss reduction's sums and counter;
// per tile its slot in the order; per segment of ORDER_SEG tiles its class
// counts
static size_t fused_ws_bytes(int64_t tiles)
{
    const int64_t segs = (tiles + ORDER_SEG - 1) / ORDER_SEG;
    return (size_t)(tiles * 4 * sizeof(double) + LOSS_TAIL_BYTES + tiles * sizeof(uint32_t) +
                    segs * ORDER_CLASSES * sizeof(uint32_t));
}

size_t gs_rasterize_fwd_bwd_l1_workspace_bytes(int32_t n_views, int32_t width, int32_t height)
{
    if (n_views < 1 || n_views > GS_MAX_VIEWS || width <= 0 || height <= 0) return 0;
    return fused_ws_bytes((int64_t)n_views * gs_tiles_x(width) * gs_tiles_y(height));
}

}  // extern "C"

// The launches of the pass with its workspace `ws` (arguments validated).
static gs_status fused_launch(const RasterArgs& a, const float* rec, int64_t n, const uint32_t* ranges,
                              const uint32_t* vals, const uint16_t* masks, int32_t n_views, const float* bg,
                              const float* target, float scale, float* image, float* T_final, int32_t* n_contrib,
                              float* dL_dimage, double* loss, float* grad2d, int32_t accumulate, void* ws,
                              hipStream_t s)
{
    const int64_t n_tiles = a.n_blocks / 4;
    if (!(accumulate & GS_ACCUMULATE_GRAD2D) && n > 0) {
        if (fill_u32((uint32_t*)grad2d, (uint64_t)n_views * GS_GRAD2D_ROWS * (uint64_t)n, 0u, s) != hipSuccess)
            return GS_ERR_HIP;
    }
    double* partial = (double*)ws;
    uint32_t* order = (uint32_t*)((char*)(partial + a.n_blocks) + LOSS_TAIL_BYTES);
    uint32_t* table = order + n_tiles;
    const uint32_t n_seg = (uint32_t)((n_tiles + ORDER_SEG - 1) / ORDER_SEG);
    hipLaunchKernelGGL(k_order_count, dim3(n_seg), dim3(ORDER_THREADS), 0, s, ranges, n_tiles, table);
    hipLaunchKernelGGL(k_order_place, dim3(n_seg), dim3(ORDER_THREADS), 0, s, ranges, n_tiles, table, n_seg, order);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    hipLaunchKernelGGL(k_raster_fwd_bwd_l1, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, s, rec, n, ranges,
                       vals, masks, a.cap, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2],
                       target, scale, image, T_final, n_contrib, dL_dimage, partial, grad2d, order);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    return loss_from_partials(partial, a.n_blocks, (double)scale, loss, (accumulate & GS_ACCUMULATE_LOSS) != 0, s) ==
                   hipSuccess
               ? GS_OK
               : GS_ERR_HIP;
}

static gs_status fused_args(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                            const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views,
                            int32_t row0, int32_t rows, const float* bg, const float* target, double* loss,
                            float* grad2d, int32_t accumulate, RasterArgs& a)
{
    if (!raster_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, a))
        return GS_ERR_INVALID_ARGUMENT;
    if (!target || !loss || (n > 0 && !grad2d)) return GS_ERR_INVALID_ARGUMENT;
    if (accumulate & ~(GS_ACCUMULATE_LOSS | GS_ACCUMULATE_GRAD2D)) return GS_ERR_INVALID_ARGUMENT;
    return GS_OK;
}

// The workspace of gs_rasterize_fwd_bwd_l1_noalloc: one array on each device
// the library runs on, held until the process ends. Host code never uses the
// name as an address: the device address comes from hipGetSymbolAddress,
// looked up once per device on the first call there.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)8 << 20;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

static gs_status scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return GS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GS_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GS_OK;
}

extern "C" {

gs_status gs_rasterize_fwd_bwd_l1(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                                  const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views,
                                  int32_t row0, int32_t rows, const float* bg, const float* target, float scale,
                                  float* image, float* T_final, int32_t* n_contrib, float* dL_dimage, double* loss,
                                  float* grad2d, int32_t accumulate, void* ws, size_t ws_bytes, void* stream)
{
    RasterArgs a;
    const gs_status st = fused_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, target,
                                    loss, grad2d, accumulate, a);
    if (st != GS_OK) return st;
    if (!ws || ws_bytes < fused_ws_bytes(a.n_blocks / 4)) return GS_ERR_INVALID_ARGUMENT;
    return fused_launch(a, rec, n, ranges, vals, masks, n_views, bg, target, scale, image, T_final, n_contrib,
                        dL_dimage, loss, grad2d, accumulate, ws, (hipStream_t)stream);
}

size_t gs_rasterize_fwd_bwd_l1_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

gs_status gs_rasterize_fwd_bwd_l1_noalloc(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                                          const uint16_t* masks, uint64_t capacity, const gs_camera* cams,
                                          int32_t n_views, int32_t row0, int32_t rows, const float* bg,
                                          const float* target, float scale, float* image, float* T_final,
                                          int32_t* n_contrib, float* dL_dimage, double* loss, float* grad2d,
                                          int32_t accumulate, void* stream)
{
    RasterArgs a;
    const gs_status st = fused_args(rec, n, ranges, vals, masks, capacity, cams, n_views, row0, rows, bg, target,
                                    loss, grad2d, accumulate, a);
    if (st != GS_OK) return st;
    if (fused_ws_bytes(a.n_blocks / 4) > NOALLOC_SCRATCH_BYTES) return GS_ERR_CAPACITY;
    void* ws = nullptr;
    const gs_status sa = scratch_address(&ws);
    if (sa != GS_OK) return sa;
    return fused_launch(a, rec, n, ranges, vals, masks, n_views, bg, target, scale, image, T_final, n_contrib,
                        dL_dimage, loss, grad2d, accumulate, ws, (hipStream_t)stream);
}

}  // extern "C"
