// gs_preprocess_bwd: chain rule from the 2D gradients (u, v, conic, opacity,
// colour) of every (view, Gaussian) to the 59 (SH degree 3) parameters of the
// Gaussian, summed over the views -- the Gaussian-wise half of the backward
// pass ("Gaussian-wise computations" of "On Scaling Up 3D Gaussian Splatting
// Training"; parameter set from its answer on the storage requirement).
//
// One thread per Gaussian. The forward quantities are recomputed with the same
// fixed-order code as gs_preprocess (project.h), so every decision (culling,
// guard-band clamp, colour clamp) is the forward's; the gradient arithmetic
// itself is ordinary fp32.
//
// With ADAM, the thread applies the Adam update to its Gaussian's P
// parameters as soon as their gradients are formed (the element-wise update
// of gs_adam_step, same arithmetic), so the gradient never goes through HBM
// and the parameters are read once. With a state array, a Gaussian culled in
// every view whose moments are known to be zero is skipped without a read:
// with g = m = v = 0 Adam leaves theta, m and v as they are (eps > 0), so
// only Gaussians seen at least once cost moment traffic.
#include "adam.h"
#include <algorithm>

#include "internal.h"
#include "project.h"

namespace gs {

// P is written only with ADAM (each thread its own Gaussian's elements,
// after reading them); out may then be null. With a list (compact output,
// not with ADAM): thread j takes Gaussian list[j] for j < *count and writes
// its gradient to column j of out, rows ostride apart (j < ostride; a list
// longer than ostride sets *overflow, never clears it, and writes nothing
// past it).
template <int DEG, bool ADAM>
__global__ __launch_bounds__(256) void k_preprocess_bwd(float* __restrict__ P, int64_t n, const DevCameras cams,
                                                        const ShConsts K, const uint16_t* __restrict__ rect,
                                                        const float* __restrict__ grad2d, float* __restrict__ out,
                                                        float* __restrict__ m, float* __restrict__ v,
                                                        const AdamConsts ac, const int32_t* __restrict__ skip,
                                                        uint8_t* __restrict__ state, uint8_t* __restrict__ vis_out,
                                                        const uint32_t* __restrict__ list,
                                                        const uint32_t* __restrict__ count, int64_t ostride,
                                                        int32_t* __restrict__ overflow)
{
    // no contraction: the arithmetic is the written one in both forms of the
    // kernel, so the gradient the fused update applies is the one
    // gs_preprocess_bwd writes, bit for bit
#pragma clang fp contract(off)
    constexpr int NB = (DEG + 1) * (DEG + 1);
    constexpr int ROWS = 11 + 3 * NB;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t g = tid, col = tid, cstride = n;  // the Gaussian, and where its gradient goes
    if (!ADAM && list) {
        const int64_t cnt = (int64_t)*count;
        if (tid == 0 && cnt > ostride) *overflow = 1;
        if (tid >= cnt || tid >= ostride) return;
        g = (int64_t)list[tid];
        if (g >= n) return;  // not a Gaussian (a list the caller never filled)
        cstride = ostride;
    }
    if (g >= n) return;
    if (ADAM && state) {
        // the skip flag, the rectangles and the state flag are requested
        // together: most waves of a large scene mostly outside the views end
        // here, after one round trip instead of three
        const int32_t sk = skip ? *skip : 0;
        const uint32_t st = state[g];
        bool seen = false;  // visible in some view
        for (int v = 0; v < cams.n_views; ++v) {
            const uint2 rr = *(const uint2*)(rect + 4 * ((int64_t)v * n + g));
            seen = seen || ((rr.y & 0xffffu) > (rr.x & 0xffffu) && (rr.y >> 16) > (rr.x >> 16));
        }
        if (sk != 0) return;  // the step's lists overflowed: no update
        if (!seen && st == 0) {
            if (out) {
#pragma unroll
                for (int r = 0; r < ROWS; ++r) out[(int64_t)r * n + g] = 0.f;
            }
            return;
        }
        if (seen) state[g] = 1;
    } else if (ADAM && skip && *skip != 0) {
        return;  // the step's lists overflowed: no update
    }
    if (!ADAM && vis_out) {
        // sparse output: a Gaussian culled in every view loads nothing and
        // writes only its flag (its gradient is zero, its rows stay as they are)
        bool seen = false;
        for (int v = 0; v < cams.n_views; ++v) {
            const uint2 rr = *(const uint2*)(rect + 4 * ((int64_t)v * n + g));
            seen = seen || ((rr.y & 0xffffu) > (rr.x & 0xffffu) && (rr.y >> 16) > (rr.x >> 16));
        }
        vis_out[g] = seen ? 1u : 0u;
        if (!seen) return;
    }
    const float x = P[0 * n + g], y = P[1 * n + g], z = P[2 * n + g];
    GaussLocal L;
    gauss_local(P[3 * n + g], P[4 * n + g], P[5 * n + g], P[6 * n + g], P[7 * n + g], P[8 * n + g],
                P[9 * n + g], P[10 * n + g], L);
    float sh[3 * NB];  // coefficients, loaded once for all views
#pragma unroll
    for (int k = 0; k < 3 * NB; ++k) sh[k] = P[(int64_t)(11 + k) * n + g];

    float gpx = 0.f, gpy = 0.f, gpz = 0.f, gop = 0.f;
    float gS3[9];  // dL/dSigma3, summed over the views
#pragma unroll
    for (int i = 0; i < 9; ++i) gS3[i] = 0.f;
    float gsh[3 * NB];
#pragma unroll
    for (int i = 0; i < 3 * NB; ++i) gsh[i] = 0.f;
    bool any = false;

    for (int v = 0; v < cams.n_views; ++v) {
        const int64_t idx = (int64_t)v * n + g;
        const uint2 rr = *(const uint2*)(rect + 4 * idx);
        if ((rr.y & 0xffffu) <= (rr.x & 0xffffu) || (rr.y >> 16) <= (rr.x >> 16)) continue;  // culled
        any = true;
        const DevCamera& cam = cams.c[v];
        ViewProj p;
        view_project(x, y, z, L, cam, cams.tiles_x, cams.tiles_y, p);
        const float* g2 = grad2d + idx * GS_GRAD2D_ROWS;  // one 36-byte record
        const float gu = g2[0], gv = g2[1], gA = g2[2], gB = g2[3], gC = g2[4];
        const float go = g2[5];
        const float grgb[3] = {g2[6], g2[7], g2[8]};
        gop += go;

        // conic Q = Sigma2^-1: dL/dSigma2 = -Q G Q, G = [[gA, gB/2], [gB/2, gC]].
        // In fp64: for a needle-like footprint Q is nearly singular and the
        // products cancel by orders of magnitude; fp32 here would cost the
        // rotation gradient (which depends on the small components) most of
        // its digits. The result is rounded back to fp32.
        const double qA = p.A, qB = p.B, qC = p.C;
        const double hB = 0.5 * (double)gB;
        const double X00 = (double)gA * qA + hB * qB, X01 = (double)gA * qB + hB * qC;
        const double X10 = hB * qA + (double)gC * qB, X11 = hB * qB + (double)gC * qC;
        const float ga = (float)(-(qA * X00 + qB * X10));
        const float gc = (float)(-(qB * X01 + qC * X11));
        const float s01 = (float)(-0.5 * ((qA * X01 + qB * X11) + (qB * X00 + qC * X10)));
        // Sigma2 = T Sigma3 T^T (+ 0.3 I): dSigma3 = T^T G2 T, dT = 2 G2 T Sigma3
        float Yt[6];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            Yt[k] = ga * p.T[k] + s01 * p.T[3 + k];
            Yt[3 + k] = s01 * p.T[k] + gc * p.T[3 + k];
        }
        float dS3[9];
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int l = 0; l < 3; ++l) dS3[3 * k + l] = p.T[k] * Yt[l] + p.T[3 + k] * Yt[3 + l];
        float TS[6];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 3; ++k)
                TS[3 * i + k] = p.T[3 * i] * L.S3[k] + p.T[3 * i + 1] * L.S3[3 + k] + p.T[3 * i + 2] * L.S3[6 + k];
        float dT[6];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            dT[k] = 2.f * (ga * TS[k] + s01 * TS[3 + k]);
            dT[3 + k] = 2.f * (s01 * TS[k] + gc * TS[3 + k]);
        }
#pragma unroll
        for (int i = 0; i < 9; ++i) gS3[i] += dS3[i];
        // T = J W
        const float* W = cam.R;
        const float dJ00 = dT[0] * W[0] + dT[1] * W[1] + dT[2] * W[2];
        const float dJ02 = dT[0] * W[6] + dT[1] * W[7] + dT[2] * W[8];
        const float dJ11 = dT[3] * W[3] + dT[4] * W[4] + dT[5] * W[5];
        const float dJ12 = dT[3] * W[6] + dT[4] * W[7] + dT[5] * W[8];
        // projected mean and Jacobian -> camera-space mean
        const float zi = 1.f / p.zc, zi2 = zi * zi, zi3 = zi2 * zi;
        float dxc = gu * cam.fx * zi;
        float dyc = gv * cam.fy * zi;
        float dzc = -(gu * cam.fx * p.xc + gv * cam.fy * p.yc) * zi2;
        dzc -= (dJ00 * cam.fx + dJ11 * cam.fy) * zi2;
        if (p.clx) {  // J02 = -fx L / z with L the clamped x/z
            dzc += dJ02 * cam.fx * p.Lx * zi2;
        } else {
            dxc -= dJ02 * cam.fx * zi2;
            dzc += 2.f * dJ02 * cam.fx * p.xc * zi3;
        }
        if (p.cly) {
            dzc += dJ12 * cam.fy * p.Ly * zi2;
        } else {
            dyc -= dJ12 * cam.fy * zi2;
            dzc += 2.f * dJ12 * cam.fy * p.yc * zi3;
        }
        gpx += W[0] * dxc + W[3] * dyc + W[6] * dzc;
        gpy += W[1] * dxc + W[4] * dyc + W[7] * dzc;
        gpz += W[2] * dxc + W[5] * dyc + W[8] * dzc;

        // colour: coefficients and view direction
        float d[3], dist;
        view_dir(x, y, z, cam, d, dist);
        float Yb[16];
        sh_eval_basis(K, DEG, d, Yb);
        float gcol[3];
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            bool clamped;
            (void)sh_channel_reg<NB>(sh, ch, Yb, clamped);
            gcol[ch] = clamped ? 0.f : grgb[ch];
        }
        float e[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const float c0 = sh[3 * k], c1 = sh[3 * k + 1], c2 = sh[3 * k + 2];
            e[k] = gcol[0] * c0 + gcol[1] * c1 + gcol[2] * c2;
            gsh[3 * k] += Yb[k] * gcol[0];
            gsh[3 * k + 1] += Yb[k] * gcol[1];
            gsh[3 * k + 2] += Yb[k] * gcol[2];
        }
        float gdx = 0.f, gdy = 0.f, gdz = 0.f;
        const float dx_ = d[0], dy_ = d[1], dz_ = d[2];
        if (DEG >= 1) {
            gdy -= K.c1 * e[1];
            gdz += K.c1 * e[2 % NB];
            gdx -= K.c1 * e[3 % NB];
        }
        if (DEG >= 2) {
            const float xx = dx_ * dx_, yy = dy_ * dy_, zz = dz_ * dz_;
            gdx += K.c2a * dy_ * e[4 % NB] - 2.f * K.c2b * dx_ * e[6 % NB] - K.c2a * dz_ * e[7 % NB] +
                   2.f * K.c2c * dx_ * e[8 % NB];
            gdy += K.c2a * dx_ * e[4 % NB] - K.c2a * dz_ * e[5 % NB] - 2.f * K.c2b * dy_ * e[6 % NB] -
                   2.f * K.c2c * dy_ * e[8 % NB];
            gdz += -K.c2a * dy_ * e[5 % NB] + 4.f * K.c2b * dz_ * e[6 % NB] - K.c2a * dx_ * e[7 % NB];
            if (DEG >= 3) {
                const float xy = dx_ * dy_, yz = dy_ * dz_, xz = dx_ * dz_;
                gdx += -6.f * K.c3a * xy * e[9 % NB] + K.c3b * yz * e[10 % NB] + 2.f * K.c3c * xy * e[11 % NB] -
                       6.f * K.c3d * xz * e[12 % NB] - K.c3c * (4.f * zz - 3.f * xx - yy) * e[13 % NB] +
                       2.f * K.c3e * xz * e[14 % NB] - K.c3a * (3.f * xx - 3.f * yy) * e[15 % NB];
                gdy += -K.c3a * (3.f * xx - 3.f * yy) * e[9 % NB] + K.c3b * xz * e[10 % NB] -
                       K.c3c * (4.f * zz - xx - 3.f * yy) * e[11 % NB] - 6.f * K.c3d * yz * e[12 % NB] +
                       2.f * K.c3c * xy * e[13 % NB] - 2.f * K.c3e * yz * e[14 % NB] + 6.f * K.c3a * xy * e[15 % NB];
                gdz += K.c3b * xy * e[10 % NB] - 8.f * K.c3c * yz * e[11 % NB] +
                       K.c3d * (6.f * zz - 3.f * xx - 3.f * yy) * e[12 % NB] - 8.f * K.c3c * xz * e[13 % NB] +
                       K.c3e * (xx - yy) * e[14 % NB];
            }
        }
        // d = (p - c) / |p - c|: project out the radial part
        const float dg = dx_ * gdx + dy_ * gdy + dz_ * gdz;
        const float inv = 1.f / dist;
        gpx += (gdx - dx_ * dg) * inv;
        gpy += (gdy - dy_ * dg) * inv;
        gpz += (gdz - dz_ * dg) * inv;
    }

    float G[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) G[r] = 0.f;
    if (any) {
        G[0] = gpx;
        G[1] = gpy;
        G[2] = gpz;
        // Sigma3 = R diag(d) R^T with d = s^2. In the rotated frame,
        // G' = R^T dL/dSigma3 R: d/d log s_j = 2 d_j G'_jj, and a rotation
        // R -> R (I + [w]x) changes L by g . w with
        // g = ((d1 - d2) (G'12 + G'21), (d2 - d0) (G'20 + G'02), (d0 - d1) (G'01 + G'10)).
        // The scale differences appear as explicit factors, computed as
        // (s_i - s_j)(s_i + s_j): a Gaussian with two nearly equal scales keeps
        // the full relative precision of its (small) gradient about that axis.
        const float* Rm = L.Rm;
        float Y[9];  // dL/dSigma3 R
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
                Y[3 * i + j] = gS3[3 * i] * Rm[j] + gS3[3 * i + 1] * Rm[3 + j] + gS3[3 * i + 2] * Rm[6 + j];
        float Gp[9];  // R^T dL/dSigma3 R
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) Gp[3 * a + b] = Rm[a] * Y[b] + Rm[3 + a] * Y[3 + b] + Rm[6 + a] * Y[6 + b];
        const float s0 = L.s[0], s1 = L.s[1], s2 = L.s[2];
        G[3] = 2.f * (s0 * s0) * Gp[0];
        G[4] = 2.f * (s1 * s1) * Gp[4];
        G[5] = 2.f * (s2 * s2) * Gp[8];
        const float om0 = ((s1 - s2) * (s1 + s2)) * (Gp[5] + Gp[7]);
        const float om1 = ((s2 - s0) * (s2 + s0)) * (Gp[6] + Gp[2]);
        const float om2 = ((s0 - s1) * (s0 + s1)) * (Gp[1] + Gp[3]);
        // unit quaternion (w, v): the body rotation w = 2 vec(conj(q^) dq^),
        // and dq^ = (I - q^ q^T) dq / |q| (the radial part drops out of it)
        if (L.qn > 0.f) {
            const float w = L.q[0], qx = L.q[1], qy = L.q[2], qz = L.q[3];
            const float k = 2.f / L.qn;
            G[6] = -k * (qx * om0 + qy * om1 + qz * om2);
            G[7] = k * (w * om0 + (qy * om2 - qz * om1));
            G[8] = k * (w * om1 + (qz * om0 - qx * om2));
            G[9] = k * (w * om2 + (qx * om1 - qy * om0));
        }
        G[10] = gop * L.o * (1.f - L.o);
#pragma unroll
        for (int i = 0; i < 3 * NB; ++i) G[11 + i] = gsh[i];
    }
    if (!ADAM || out) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) out[(int64_t)r * cstride + col] = G[r];
    }
    if (ADAM) {
        // the parameters still in registers (position, SH) are not read
        // again; the moments of CH rows are requested before any is used, so
        // that each wave keeps many loads in flight. Moments and parameters
        // stream through with nontemporal loads and stores: kept in the
        // caches as dirty lines, the 708 bytes per Gaussian were written back
        // while the next step's preprocess ran, and slowed it
        constexpr int CH = 20;
#pragma unroll
        for (int r0 = 0; r0 < ROWS; r0 += CH) {
            float mm[CH], vv[CH], pp[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int r = r0 + c;
                if (r < ROWS) {
                    const int64_t e = (int64_t)r * n + g;
                    mm[c] = __builtin_nontemporal_load(m + e);
                    vv[c] = __builtin_nontemporal_load(v + e);
                    pp[c] = r == 0 ? x : r == 1 ? y : r == 2 ? z : r >= 11 ? sh[r - 11] : P[e];
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int r = r0 + c;
                if (r < ROWS) {
                    const int64_t e = (int64_t)r * n + g;
                    adam1(pp[c], G[r], mm[c], vv[c], ac);
                    __builtin_nontemporal_store(pp[c], P + e);
                    __builtin_nontemporal_store(mm[c], m + e);
                    __builtin_nontemporal_store(vv[c], v + e);
                }
            }
        }
    }
}

template <bool ADAM>
static gs_status pbwd_launch(float* params, int64_t n, int32_t sh_degree, const DevCameras& dc,
                             const uint16_t* rect, const float* grad2d, float* out, float* m, float* v,
                             const AdamConsts& c, const int32_t* skip, uint8_t* state, uint8_t* vis_out, hipStream_t s,
                             const uint32_t* list = nullptr, const uint32_t* count = nullptr, int64_t ostride = 0,
                             int32_t* overflow = nullptr)
{
    // with a list, one thread per possible list entry: at most min(n, ostride)
    const int64_t threads = list ? std::min<int64_t>(n, ostride) : n;
    const dim3 grid(grid_for((uint64_t)std::max<int64_t>(threads, 1), 256)), block(256);
    const ShConsts K = sh_constants();
    switch (sh_degree) {
        case 0: hipLaunchKernelGGL((k_preprocess_bwd<0, ADAM>), grid, block, 0, s, params, n, dc, K, rect, grad2d, out, m, v, c, skip, state, vis_out, list, count, ostride, overflow); break;
        case 1: hipLaunchKernelGGL((k_preprocess_bwd<1, ADAM>), grid, block, 0, s, params, n, dc, K, rect, grad2d, out, m, v, c, skip, state, vis_out, list, count, ostride, overflow); break;
        case 2: hipLaunchKernelGGL((k_preprocess_bwd<2, ADAM>), grid, block, 0, s, params, n, dc, K, rect, grad2d, out, m, v, c, skip, state, vis_out, list, count, ostride, overflow); break;
        default: hipLaunchKernelGGL((k_preprocess_bwd<3, ADAM>), grid, block, 0, s, params, n, dc, K, rect, grad2d, out, m, v, c, skip, state, vis_out, list, count, ostride, overflow); break;
    }
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_preprocess_bwd(const float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                            int32_t n_views, const uint16_t* rect, const float* grad2d, float* grad_params,
                            uint8_t* visible, void* stream)
{
    if (n < 0 || sh_degree < 0 || sh_degree > 3) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !rect || !grad2d || !grad_params)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    DevCameras dc;
    if (!make_dev_cameras(cams, n_views, dc)) return GS_ERR_INVALID_ARGUMENT;
    if (n == 0) return GS_OK;
    return pbwd_launch<false>((float*)params, n, sh_degree, dc, rect, grad2d, grad_params, nullptr, nullptr,
                              AdamConsts{}, nullptr, nullptr, visible, (hipStream_t)stream);
}

gs_status gs_preprocess_bwd_compact(const float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                                    int32_t n_views, const uint16_t* rect, const float* grad2d,
                                    const uint32_t* list, const uint32_t* count, int64_t stride,
                                    float* grad_compact, int32_t* overflow, void* stream)
{
    if (n < 0 || sh_degree < 0 || sh_degree > 3 || stride < 1) return GS_ERR_INVALID_ARGUMENT;
    if (!list || !count || !grad_compact || !overflow) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !rect || !grad2d)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31) || stride > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    DevCameras dc;
    if (!make_dev_cameras(cams, n_views, dc)) return GS_ERR_INVALID_ARGUMENT;
    if (n == 0) return GS_OK;
    return pbwd_launch<false>((float*)params, n, sh_degree, dc, rect, grad2d, grad_compact, nullptr, nullptr,
                              AdamConsts{}, nullptr, nullptr, nullptr, (hipStream_t)stream, list, count, stride,
                              overflow);
}

gs_status gs_preprocess_bwd_adam(float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                                 int32_t n_views, const uint16_t* rect, const float* grad2d, float* m, float* v,
                                 double lr, double beta1, double beta2, double eps, int64_t step,
                                 const int32_t* skip, uint8_t* state, float* grad_params, void* stream)
{
    if (n < 0 || sh_degree < 0 || sh_degree > 3) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!params || !rect || !grad2d || !m || !v)) return GS_ERR_INVALID_ARGUMENT;
    if (n > ((int64_t)1 << 31)) return GS_ERR_INVALID_ARGUMENT;
    DevCameras dc;
    if (!make_dev_cameras(cams, n_views, dc)) return GS_ERR_INVALID_ARGUMENT;
    AdamConsts c;
    if (!adam_consts(lr, beta1, beta2, eps, step, c)) return GS_ERR_INVALID_ARGUMENT;
    if (n == 0) return GS_OK;
    return pbwd_launch<true>(params, n, sh_degree, dc, rect, grad2d, grad_params, m, v, c, skip, state, nullptr,
                             (hipStream_t)stream);
}

}  // extern "C"
