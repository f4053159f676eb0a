// gs_loss_l1 and gs_adam_step: element-wise streaming kernels (HBM-bound).
//
// L1 loss with views averaged ("On Scaling Up 3D Gaussian Splatting
// Training", answer on the Independent Gradients Hypothesis: gradients
// averaged over the views of a batch); Adam of Kingma & Ba (reference [12] of
// "A Scalable PyTorch Abstraction for Multi-GPU Gaussian Splatting") with the
// two moment vectors that make up 708 bytes per Gaussian ("AMD ROCm team
// open-sources distributed 3D Gaussian Splatting...", section "Distributed
// training architecture and memory scaling").
#include <math.h>

#include <algorithm>

#include "adam.h"
#include "internal.h"

namespace gs {

constexpr int EW_THREADS = 256;

__global__ __launch_bounds__(EW_THREADS) void k_loss_l1(const float* __restrict__ image,
                                                        const float* __restrict__ target, int64_t count,
                                                        float scale, float* __restrict__ dL,
                                                        double* __restrict__ loss)
{
    __shared__ double s_part[EW_THREADS / 64];
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS * 4;
    double acc = 0.0;
    for (int64_t base = ((int64_t)blockIdx.x * EW_THREADS + threadIdx.x) * 4; base < count; base += stride) {
        if (base + 4 <= count) {
            const float4 a = *(const float4*)(image + base), b = *(const float4*)(target + base);
            const float d0 = a.x - b.x, d1 = a.y - b.y, d2 = a.z - b.z, d3 = a.w - b.w;
            acc += (double)(fabsf(d0) + fabsf(d1)) + (double)(fabsf(d2) + fabsf(d3));
            *(float4*)(dL + base) =
                make_float4(d0 > 0.f ? scale : (d0 < 0.f ? -scale : 0.f), d1 > 0.f ? scale : (d1 < 0.f ? -scale : 0.f),
                            d2 > 0.f ? scale : (d2 < 0.f ? -scale : 0.f), d3 > 0.f ? scale : (d3 < 0.f ? -scale : 0.f));
        } else {
            for (int64_t i = base; i < count; ++i) {
                const float d = image[i] - target[i];
                acc += (double)fabsf(d);
                dL[i] = d > 0.f ? scale : (d < 0.f ? -scale : 0.f);
            }
        }
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < EW_THREADS / 64; ++w) t += s_part[w];
        atomicAdd(loss, t * (double)scale);
    }
}

__global__ __launch_bounds__(EW_THREADS) void k_adam(float* __restrict__ params, const float* __restrict__ grad,
                                                     float* __restrict__ m, float* __restrict__ v, int64_t count,
                                                     const AdamConsts c, const int32_t* __restrict__ skip)
{
    if (skip && *skip != 0) return;  // the step's lists overflowed: no update
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS * 4;
    for (int64_t base = ((int64_t)blockIdx.x * EW_THREADS + threadIdx.x) * 4; base < count; base += stride) {
        if (base + 4 <= count) {
            float4 p = *(float4*)(params + base), mm = *(float4*)(m + base), vv = *(float4*)(v + base);
            const float4 g = *(const float4*)(grad + base);
            adam1(p.x, g.x, mm.x, vv.x, c);
            adam1(p.y, g.y, mm.y, vv.y, c);
            adam1(p.z, g.z, mm.z, vv.z, c);
            adam1(p.w, g.w, mm.w, vv.w, c);
            *(float4*)(params + base) = p;
            *(float4*)(m + base) = mm;
            *(float4*)(v + base) = vv;
        } else {
            for (int64_t i = base; i < count; ++i) adam1(params[i], grad[i], m[i], v[i], c);
        }
    }
}

// Adam over a [P][n] block where only the Gaussians with visible[g] set have a
// gradient (the sparse output of gs_preprocess_bwd): one thread per Gaussian,
// its P elements one row after the other (consecutive threads, consecutive
// elements of a row). A Gaussian without a gradient reads no gradient (g = 0:
// its moments decay and its parameters move by the decayed moments); with
// state flags, one whose moments are known to be zero is skipped (its update
// is the identity when eps > 0).
constexpr int AV_CHUNK = 16;

__global__ __launch_bounds__(EW_THREADS) void k_adam_visible(float* __restrict__ params, const float* __restrict__ grad,
                                                             float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                             int32_t P, const uint8_t* __restrict__ visible,
                                                             uint8_t* __restrict__ state, const AdamConsts c,
                                                             const int32_t* __restrict__ skip)
{
    const int64_t g = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x;
    if (g >= n) return;
    if (skip && *skip != 0) return;  // the step's lists overflowed: no update
    const bool vis = visible[g] != 0;
    if (state) {
        if (!vis && state[g] == 0) return;
        if (vis) state[g] = 1;
    }
    for (int r0 = 0; r0 < P; r0 += AV_CHUNK) {
        float pp[AV_CHUNK], mm[AV_CHUNK], vv[AV_CHUNK], gg[AV_CHUNK];
#pragma unroll
        for (int k = 0; k < AV_CHUNK; ++k) {
            const int r = r0 + k;
            if (r < P) {
                const int64_t e = (int64_t)r * n + g;
                pp[k] = params[e];
                mm[k] = m[e];
                vv[k] = v[e];
                gg[k] = vis ? grad[e] : 0.f;
            }
        }
#pragma unroll
        for (int k = 0; k < AV_CHUNK; ++k) {
            const int r = r0 + k;
            if (r < P) {
                const int64_t e = (int64_t)r * n + g;
                adam1(pp[k], gg[k], mm[k], vv[k], c);
                params[e] = pp[k];
                m[e] = mm[k];
                v[e] = vv[k];
            }
        }
    }
}

// Adam from a compact gradient: k_adam_listed updates the Gaussians of the
// list (list[j] with its gradient in column j of grad, rows `stride` apart;
// j < min(*count, stride)), AL_ROWS rows of one Gaussian per thread, the grid's
// y dimension over the row groups (more independent loads in flight than one
// thread walking all rows: city block 1.14 -> 1.09 ms); k_adam_unlisted applies
// the update of a zero gradient to every other Gaussian (one that no view
// sees: the list holds exactly those some view sees), or, with state flags,
// only to those whose moments may be non-zero. Same arithmetic as k_adam, so
// the same bits as the dense update of the dense gradient.
constexpr int AL_ROWS = 4;
constexpr int AL_MAX_ROWS = 65535 * AL_ROWS;  // the grid's y dimension

__global__ __launch_bounds__(EW_THREADS) void k_adam_listed(float* __restrict__ params, const float* __restrict__ grad,
                                                            int64_t stride, const uint32_t* __restrict__ list,
                                                            const uint32_t* __restrict__ count,
                                                            float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                            int32_t P, uint8_t* __restrict__ state,
                                                            const AdamConsts c, const int32_t* __restrict__ skip)
{
    const int64_t j = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x;
    if (j >= stride || j >= (int64_t)*count) return;
    if (skip && *skip != 0) return;  // the step's lists overflowed: no update
    const int64_t g = (int64_t)list[j];
    if (g >= n) return;
    const int r0 = (int)blockIdx.y * AL_ROWS;
    if (state && r0 == 0) state[g] = 1;
    float pp[AL_ROWS], mm[AL_ROWS], vv[AL_ROWS], gg[AL_ROWS];
#pragma unroll
    for (int k = 0; k < AL_ROWS; ++k) {
        const int r = r0 + k;
        if (r < P) {
            const int64_t e = (int64_t)r * n + g;
            pp[k] = params[e];
            mm[k] = m[e];
            vv[k] = v[e];
            gg[k] = grad[(int64_t)r * stride + j];
        }
    }
#pragma unroll
    for (int k = 0; k < AL_ROWS; ++k) {
        const int r = r0 + k;
        if (r < P) {
            const int64_t e = (int64_t)r * n + g;
            adam1(pp[k], gg[k], mm[k], vv[k], c);
            params[e] = pp[k];
            m[e] = mm[k];
            v[e] = vv[k];
        }
    }
}

__global__ __launch_bounds__(EW_THREADS) void k_adam_unlisted(float* __restrict__ params, float* __restrict__ m,
                                                              float* __restrict__ v, int64_t n, int32_t P,
                                                              const uint16_t* __restrict__ rect, int32_t n_views,
                                                              const uint8_t* __restrict__ state, const AdamConsts c,
                                                              const int32_t* __restrict__ skip)
{
    const int64_t g = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x;
    if (g >= n) return;
    const int32_t sk = skip ? *skip : 0;
    const uint32_t st = state ? state[g] : 1u;
    bool seen = false;
    for (int vw = 0; vw < n_views; ++vw) {
        const uint2 rr = *(const uint2*)(rect + 4 * ((int64_t)vw * n + g));
        seen = seen || ((rr.y & 0xffffu) > (rr.x & 0xffffu) && (rr.y >> 16) > (rr.x >> 16));
    }
    if (sk != 0 || seen || st == 0u) return;  // no update, a listed Gaussian, or moments known zero
    for (int r = 0; r < P; ++r) {
        const int64_t e = (int64_t)r * n + g;
        float pp = params[e], mm = m[e], vv = v[e];
        adam1(pp, 0.f, mm, vv, c);
        params[e] = pp;
        m[e] = mm;
        v[e] = vv;
    }
}

// Enough blocks to fill the chip several times over; each thread then walks
// its grid-stride range. The loss uses fewer blocks: each block ends with one
// fp64 atomic on the same address.
static unsigned stream_blocks(int64_t count, int64_t cap = 256 * 32)
{
    const int64_t need = (count / 4 + EW_THREADS - 1) / EW_THREADS;
    return (unsigned)(need < 1 ? 1 : (need > cap ? cap : need));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_loss_l1(const float* image, const float* target, int64_t count, float scale, float* dL_dimage,
                     double* loss, int32_t accumulate, void* stream)
{
    if (count < 0 || !loss) return GS_ERR_INVALID_ARGUMENT;
    if (count > 0 && (!image || !target || !dL_dimage)) return GS_ERR_INVALID_ARGUMENT;
    if (!aligned16(image) || !aligned16(target) || !aligned16(dL_dimage)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate && fill_u32((uint32_t*)loss, 2, 0u, s) != hipSuccess) return GS_ERR_HIP;
    if (count == 0) return GS_OK;
    hipLaunchKernelGGL(k_loss_l1, dim3(stream_blocks(count, 256 * 4)), dim3(EW_THREADS), 0, s, image, target,
                       count, scale, dL_dimage, loss);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

static gs_status adam_launch(float* params, const float* grad, float* m, float* v, int64_t count, double lr,
                             double beta1, double beta2, double eps, int64_t step, const int32_t* skip, void* stream)
{
    if (count < 0 || step < 1) return GS_ERR_INVALID_ARGUMENT;
    if (count > 0 && (!params || !grad || !m || !v)) return GS_ERR_INVALID_ARGUMENT;
    if (!aligned16(params) || !aligned16(grad) || !aligned16(m) || !aligned16(v)) return GS_ERR_INVALID_ARGUMENT;
    if (count == 0) return GS_OK;
    AdamConsts c;
    if (!adam_consts(lr, beta1, beta2, eps, step, c)) return GS_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(k_adam, dim3(stream_blocks(count)), dim3(EW_THREADS), 0, (hipStream_t)stream, params, grad, m,
                       v, count, c, skip);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_adam_step(float* params, const float* grad, float* m, float* v, int64_t count, double lr, double beta1,
                       double beta2, double eps, int64_t step, void* stream)
{
    return adam_launch(params, grad, m, v, count, lr, beta1, beta2, eps, step, nullptr, stream);
}

gs_status gs_adam_step_visible(float* params, const float* grad, float* m, float* v, int64_t n, int32_t rows,
                               const uint8_t* visible, uint8_t* state, double lr, double beta1, double beta2,
                               double eps, int64_t step, const int32_t* skip, void* stream)
{
    if (n < 0 || rows < 1 || step < 1) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !grad || !m || !v || !visible)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    AdamConsts c;
    if (!adam_consts(lr, beta1, beta2, eps, step, c)) return GS_ERR_INVALID_ARGUMENT;
    if (state && !(eps > 0.0)) return GS_ERR_INVALID_ARGUMENT;  // with eps = 0 the skipped update is 0/0, not the identity
    if (n == 0) return GS_OK;
    hipLaunchKernelGGL(k_adam_visible, dim3((unsigned)((n + EW_THREADS - 1) / EW_THREADS)), dim3(EW_THREADS), 0,
                       (hipStream_t)stream, params, grad, m, v, n, rows, visible, state, c, skip);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_adam_step_compact(float* params, const float* grad_compact, int64_t stride, const uint32_t* list,
                               const uint32_t* count, float* m, float* v, int64_t n, int32_t rows,
                               const uint16_t* rect, int32_t n_views, uint8_t* state, double lr, double beta1,
                               double beta2, double eps, int64_t step, const int32_t* skip, void* stream)
{
    if (n < 0 || rows < 1 || rows > AL_MAX_ROWS || step < 1 || stride < 1 || n_views < 1 || n_views > GS_MAX_VIEWS)
        return GS_ERR_INVALID_ARGUMENT;
    if (!list || !count || !grad_compact) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !m || !v || !rect)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31) || stride > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    AdamConsts c;
    if (!adam_consts(lr, beta1, beta2, eps, step, c)) return GS_ERR_INVALID_ARGUMENT;
    if (state && !(eps > 0.0)) return GS_ERR_INVALID_ARGUMENT;  // with eps = 0 the skipped update is 0/0, not the identity
    if (n == 0) return GS_OK;
    hipStream_t s = (hipStream_t)stream;
    // the unlisted first: it reads the state flags before the listed pass sets them
    hipLaunchKernelGGL(k_adam_unlisted, dim3((unsigned)((n + EW_THREADS - 1) / EW_THREADS)), dim3(EW_THREADS), 0, s,
                       params, m, v, n, rows, rect, n_views, state, c, skip);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    const int64_t lj = std::min<int64_t>(n, stride);
    const dim3 lgrid((unsigned)((lj + EW_THREADS - 1) / EW_THREADS), (unsigned)((rows + AL_ROWS - 1) / AL_ROWS));
    hipLaunchKernelGGL(k_adam_listed, lgrid, dim3(EW_THREADS), 0, s,
                       params, grad_compact, stride, list, count, m, v, n, rows, state, c, skip);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

gs_status gs_adam_step_unless(float* params, const float* grad, float* m, float* v, int64_t count, double lr,
                              double beta1, double beta2, double eps, int64_t step, const int32_t* skip, void* stream)
{
    if (!skip) return GS_ERR_INVALID_ARGUMENT;
    return adam_launch(params, grad, m, v, count, lr, beta1, beta2, eps, step, skip, stream);
}

}  // extern "C"
