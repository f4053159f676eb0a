// Device-side helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"

#define GS_WAVE 64

// Camera as the kernels see it (passed by value in the kernel arguments).
struct DevCamera {
    float R[9];
    float t[3];
    float fx, fy, cx, cy;
    float near_plane, far_plane;
    float limx, limy;  // guard band of the EWA Jacobian on x/z, y/z
    float ccx, ccy, ccz;  // camera centre in world space
};

struct DevCameras {
    DevCamera c[GS_MAX_VIEWS];
    int32_t n_views;
    int32_t width, height;
    int32_t tiles_x, tiles_y;
    int32_t tiles_per_view;
};

// Real SH constants (Condon-Shortley sign), fp32 values of their closed forms.
struct ShConsts {
    float c0, c1, c2a, c2b, c2c, c3a, c3b, c3c, c3d, c3e;
};

// The blocks of a launch are dealt round-robin to the 8 XCDs (block b runs on
// XCD b % 8). Renumber so that each XCD receives one contiguous range of
// logical blocks: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t nblocks)
{
    const uint32_t xcd = bid & 7u, idx = bid >> 3;
    const uint32_t per = nblocks >> 3, rem = nblocks & 7u;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t mask_rank(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Sum over the 64 lanes with DPP row operations; every lane returns the total.
__device__ __forceinline__ float wave_sum(float x)
{
    // within each row of 16 lanes
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false)); // row_half_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false)); // row_mirror
    // across the four rows
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_max(float x)
{
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ int wave_max_int(int x)
{
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
    return x;
}

#define GS_CHECK_LAUNCH()                                   \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP; \
    } while (0)
