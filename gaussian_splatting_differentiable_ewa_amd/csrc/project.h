// Gaussian-wise projection shared by the forward (preprocess) and backward
// (preprocess_bwd) kernels: activations, EWA 2D covariance, radius, tile
// rectangle and SH colour.
//
// Every quantity here feeds an integer result (culling, radius, rectangle,
// depth key) or a clamp decision, so it is evaluated in one fixed fp32 order:
// contraction of a*b+c into fma is off in this header (see the pragmas), and
// division and sqrt are IEEE-rounded. exp() of a log-scale and the sigmoid
// are evaluated in fp64 and rounded once.
//
// The formulas are the EWA splatting form of the 3DGS method (reference [10]
// of "A Scalable PyTorch Abstraction for Multi-GPU Gaussian Splatting"): a 3D
// covariance R diag(s)^2 R^T from a unit quaternion and log-scales, projected
// with the Jacobian of the perspective map at the mean, plus a 0.3 px^2
// screen-space low-pass filter; tiles of 16x16 pixels ("On Scaling Up 3D
// Gaussian Splatting Training", answer (1) on pixel block size).
#pragma once

#include "common.h"

struct GaussLocal {
    float s[3];      // scales
    float o;         // opacity
    float q[4];      // unit quaternion w x y z
    float qn;        // norm of the raw quaternion (0 -> identity)
    float Rm[9];     // rotation, row-major
    float M[9];      // R diag(s)
    float S3[9];     // M M^T
};

__device__ __forceinline__ void gauss_local(float ls0, float ls1, float ls2, float qw, float qx,
                                            float qy, float qz, float logit, GaussLocal& L)
{
#pragma clang fp contract(off)
    L.s[0] = (float)exp((double)ls0);
    L.s[1] = (float)exp((double)ls1);
    L.s[2] = (float)exp((double)ls2);
    L.o = (float)(1.0 / (1.0 + exp(-(double)logit)));
    const float nrm = sqrtf(((qw * qw + qx * qx) + qy * qy) + qz * qz);
    L.qn = nrm;
    if (nrm > 0.f) {
        L.q[0] = qw / nrm; L.q[1] = qx / nrm; L.q[2] = qy / nrm; L.q[3] = qz / nrm;
    } else {
        L.q[0] = 1.f; L.q[1] = 0.f; L.q[2] = 0.f; L.q[3] = 0.f;
    }
    const float w = L.q[0], x = L.q[1], y = L.q[2], z = L.q[3];
    L.Rm[0] = 1.f - 2.f * (y * y + z * z);
    L.Rm[1] = 2.f * (x * y - w * z);
    L.Rm[2] = 2.f * (x * z + w * y);
    L.Rm[3] = 2.f * (x * y + w * z);
    L.Rm[4] = 1.f - 2.f * (x * x + z * z);
    L.Rm[5] = 2.f * (y * z - w * x);
    L.Rm[6] = 2.f * (x * z - w * y);
    L.Rm[7] = 2.f * (y * z + w * x);
    L.Rm[8] = 1.f - 2.f * (x * x + y * y);
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) L.M[3 * i + j] = L.Rm[3 * i + j] * L.s[j];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            L.S3[3 * i + j] = (L.M[3 * i] * L.M[3 * j] + L.M[3 * i + 1] * L.M[3 * j + 1]) +
                              L.M[3 * i + 2] * L.M[3 * j + 2];
}

struct ViewProj {
    float xc, yc, zc;
    bool clx, cly;           // guard-band clamp active on x/z, y/z
    float Lx, Ly;            // x/z and y/z after the guard-band clamp
    float J00, J02, J11, J12;
    float T[6];              // J R_cam
    float a, b, c;           // dilated 2D covariance
    float det, A, B, C;      // conic
    float u, v, rad;
    int x0, y0, x1, y1;
    bool visible;
};

// Camera transform, EWA covariance, conic, radius and tile rectangle of one
// Gaussian in one view. Fills `p` up to the first failed test; p.visible says
// whether the pair survives.
__device__ __forceinline__ void view_project(float x, float y, float z, const GaussLocal& L,
                                             const DevCamera& cam, int TX, int TY, ViewProj& p)
{
#pragma clang fp contract(off)
    const float* W = cam.R;
    p.visible = false;
    p.xc = ((W[0] * x + W[1] * y) + W[2] * z) + cam.t[0];
    p.yc = ((W[3] * x + W[4] * y) + W[5] * z) + cam.t[1];
    p.zc = ((W[6] * x + W[7] * y) + W[8] * z) + cam.t[2];
    const float zc = p.zc;
    if (!(zc > cam.near_plane && zc < cam.far_plane)) return;

    float txz = p.xc / zc, tyz = p.yc / zc;
    p.clx = false;
    p.cly = false;
    if (txz < -cam.limx) { txz = -cam.limx; p.clx = true; }
    else if (txz > cam.limx) { txz = cam.limx; p.clx = true; }
    if (tyz < -cam.limy) { tyz = -cam.limy; p.cly = true; }
    else if (tyz > cam.limy) { tyz = cam.limy; p.cly = true; }
    p.Lx = txz;
    p.Ly = tyz;
    const float tx = txz * zc, ty = tyz * zc;
    const float zz = zc * zc;
    p.J00 = cam.fx / zc;
    p.J02 = -(cam.fx * tx) / zz;
    p.J11 = cam.fy / zc;
    p.J12 = -(cam.fy * ty) / zz;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        p.T[k] = p.J00 * W[k] + p.J02 * W[6 + k];
        p.T[3 + k] = p.J11 * W[3 + k] + p.J12 * W[6 + k];
    }
    float U[6];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            U[3 * i + j] = (p.T[3 * i] * L.S3[j] + p.T[3 * i + 1] * L.S3[3 + j]) +
                           p.T[3 * i + 2] * L.S3[6 + j];
    const float a0 = (U[0] * p.T[0] + U[1] * p.T[1]) + U[2] * p.T[2];
    const float b0 = (U[0] * p.T[3] + U[1] * p.T[4]) + U[2] * p.T[5];
    const float c0 = (U[3] * p.T[3] + U[4] * p.T[4]) + U[5] * p.T[5];
    p.a = a0 + 0.3f;
    p.b = b0;
    p.c = c0 + 0.3f;
    p.det = p.a * p.c - p.b * p.b;
    if (!(p.det > 0.f)) return;
    p.A = p.c / p.det;
    p.B = -p.b / p.det;
    p.C = p.a / p.det;
    const float mid = 0.5f * (p.a + p.c);
    const float lam = mid + sqrtf(fmaxf(mid * mid - p.det, 0.f));
    p.rad = ceilf(3.f * sqrtf(lam));
    p.u = (cam.fx * p.xc) / zc + cam.cx;
    p.v = (cam.fy * p.yc) / zc + cam.cy;
    const float fTX = (float)TX, fTY = (float)TY;
    p.x0 = (int)fminf(fmaxf(floorf((p.u - p.rad) / 16.f), 0.f), fTX);
    p.x1 = (int)fminf(fmaxf(ceilf((p.u + p.rad) / 16.f), 0.f), fTX);
    p.y0 = (int)fminf(fmaxf(floorf((p.v - p.rad) / 16.f), 0.f), fTY);
    p.y1 = (int)fminf(fmaxf(ceilf((p.v + p.rad) / 16.f), 0.f), fTY);
    p.visible = (p.x1 > p.x0) && (p.y1 > p.y0);
}

// Unit direction from the camera centre to the mean (world space) and the
// distance, in the fixed order.
__device__ __forceinline__ void view_dir(float x, float y, float z, const DevCamera& cam, float d[3],
                                         float& dist)
{
#pragma clang fp contract(off)
    float dx = x - cam.ccx, dy = y - cam.ccy, dz = z - cam.ccz;
    dist = sqrtf((dx * dx + dy * dy) + dz * dz);
    d[0] = dx / dist;
    d[1] = dy / dist;
    d[2] = dz / dist;
}

// Real SH basis up to degree `deg` at unit direction d (k = l^2 + l + m).
__device__ __forceinline__ void sh_eval_basis(const ShConsts& K, int deg, const float d[3], float Y[16])
{
#pragma clang fp contract(off)
    const float x = d[0], y = d[1], z = d[2];
    Y[0] = K.c0;
    if (deg < 1) return;
    Y[1] = -(K.c1 * y);
    Y[2] = K.c1 * z;
    Y[3] = -(K.c1 * x);
    if (deg < 2) return;
    const float xx = x * x, yy = y * y, zz = z * z;
    const float xy = x * y, yz = y * z, xz = x * z;
    Y[4] = K.c2a * xy;
    Y[5] = -(K.c2a * yz);
    Y[6] = K.c2b * ((2.f * zz - xx) - yy);
    Y[7] = -(K.c2a * xz);
    Y[8] = K.c2c * (xx - yy);
    if (deg < 3) return;
    Y[9] = -(K.c3a * (y * (3.f * xx - yy)));
    Y[10] = K.c3b * (xy * z);
    Y[11] = -(K.c3c * (y * ((4.f * zz - xx) - yy)));
    Y[12] = K.c3d * (z * ((2.f * zz - 3.f * xx) - 3.f * yy));
    Y[13] = -(K.c3c * (x * ((4.f * zz - xx) - yy)));
    Y[14] = K.c3e * (z * (xx - yy));
    Y[15] = -(K.c3a * (x * (xx - 3.f * yy)));
}

// The same sum with the coefficients already in registers (sh[3k + c]).
template <int NB>
__device__ __forceinline__ float sh_channel_reg(const float* sh, int ch, const float Y[16], bool& clamped)
{
#pragma clang fp contract(off)
    float acc = Y[0] * sh[ch];
#pragma unroll
    for (int k = 1; k < NB; ++k) acc = acc + Y[k] * sh[3 * k + ch];
    acc = acc + 0.5f;
    clamped = acc < 0.f;
    return clamped ? 0.f : acc;
}

// Colour of channel c: sum_k Y_k sh[k][c] in index order, + 0.5, clamped at
// zero. `sh` points at row 11 of the parameter block, stride n.
__device__ __forceinline__ float sh_channel(const float* __restrict__ sh, int64_t n, int64_t g,
                                            int nb, int ch, const float Y[16], bool& clamped)
{
#pragma clang fp contract(off)
    float acc = Y[0] * sh[(int64_t)ch * n + g];
    for (int k = 1; k < nb; ++k) acc = acc + Y[k] * sh[(int64_t)(3 * k + ch) * n + g];
    acc = acc + 0.5f;
    clamped = acc < 0.f;
    return clamped ? 0.f : acc;
}
