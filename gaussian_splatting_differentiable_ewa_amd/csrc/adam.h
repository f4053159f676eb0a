// The Adam update of one element (Kingma & Ba, reference [12] of "A Scalable
// PyTorch Abstraction for Multi-GPU Gaussian Splatting"), shared by the
// element-wise optimizer kernel and the preprocess backward kernel that
// applies it to each Gaussian's parameters as soon as their gradient exists.
#pragma once

#include <math.h>

#include "common.h"

namespace gs {

struct AdamConsts {
    float b1, omb1, b2, omb2;  // beta and 1 - beta, each rounded once from fp64
    float eps;
    float step_size;     // lr / (1 - beta1^t)
    float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
};

// Bias corrections formed in fp64 on the host, rounded once. False for
// step < 1, beta outside [0, 1) or eps < 0.
inline bool adam_consts(double lr, double beta1, double beta2, double eps, int64_t step, AdamConsts& c)
{
    if (step < 1) return false;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0)) return false;
    const double bc1 = 1.0 - pow(beta1, (double)step);
    const double bc2 = 1.0 - pow(beta2, (double)step);
    c.b1 = (float)beta1;
    c.omb1 = (float)(1.0 - beta1);
    c.b2 = (float)beta2;
    c.omb2 = (float)(1.0 - beta2);
    c.eps = (float)eps;
    c.step_size = (float)(lr / bc1);
    c.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
    return true;
}

__device__ __forceinline__ void adam1(float& p, float g, float& m, float& v, const AdamConsts& c)
{
#pragma clang fp contract(off)  // the same rounding wherever it is inlined
    m = c.b1 * m + c.omb1 * g;
    v = c.b2 * v + c.omb2 * (g * g);
    p = p - c.step_size * m / (sqrtf(v) * c.inv_sqrt_bc2 + c.eps);
}

}  // namespace gs
