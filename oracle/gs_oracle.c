/*
 * TEST INFRASTRUCTURE ONLY -- CPU oracle of one training step of the tile-based
 * differentiable Gaussian rasterizer. It is loaded by the test suite, the smoke
 * check and the benchmark's CPU-baseline leg, never by the product path, and it
 * shares no code, header, table or constant with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 *
 * Contents:
 *   or_*_f32 / or_*_f64  precision-generic stages (gs_oracle_body.h)
 *   or_emit_sorted       intersection keys + library sort (total order)
 *   or_tile_ranges       per-tile [start, end) of the sorted list
 *   or_exclusive_scan    prefix sum of per-(view, Gaussian) tile counts
 *   or_adam              textbook Adam (Kingma & Ba, reference [12] of "A
 *                        Scalable PyTorch Abstraction for Multi-GPU Gaussian
 *                        Splatting")
 */
#define _GNU_SOURCE
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

typedef struct {
    int32_t width, height;
    float fx, fy, cx, cy;
    float R[9]; /* world -> camera rotation, row-major: p_c = R p + t */
    float t[3];
    float near_plane, far_plane;
} or_camera;

#define OR_REC 16
#define OR_INT 8

int or_abi_version(void) { return 1; }
int or_rec_stride(void) { return OR_REC; }
int or_int_stride(void) { return OR_INT; }
int or_camera_bytes(void) { return (int)sizeof(or_camera); }
int or_max_threads(void) { return omp_get_max_threads(); }
void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---------------------------------------------------------------------------
 * How far a GPU's exp() may lie from this oracle's, and so which per-pixel
 * decisions of the compositing rules (alpha >= 1/255, the 0.99 clamp, the
 * T' < 1e-4 stop) the two sides may take differently.
 *
 * A (pixel, entry) pair's power is the same fp32 arithmetic on both sides, so
 * it is the same number. The GPU's raster passes take G = exp(p) as 2^y with
 * y = fl(p * L), L = fl32(log2 e), on the hardware exp2, whose result is
 * within OR_EXP_HW_ULP ulp of 2^y; this oracle takes the C library's expf(p),
 * within OR_EXP_LIBM_REL (relative) of e^p. With
 *   dy = |p| (|L - log2 e| + L u)        (the constant's rounding and the
 *                                         product's, u = 2^-24)
 *   e_arg = 2^dy - 1                     (2^y against e^p)
 * the two G differ by at most (relative to the oracle's)
 *   rG(p) = (1 + e_arg) (1 + 2^-23 OR_EXP_HW_ULP) / (1 - OR_EXP_LIBM_REL) - 1,
 * and the two products o * G, each rounded once, by
 *   ra(p) = (1 + rG) (1 + u) / (1 - u) - 1.
 * One ulp of a normal fp32 result r is at most 2^-23 r. tests/test_oracle_band.py
 * checks rG against the exact error of the argument for every fp32 power in
 * [-5.6, 0] and the library's expf against fp64; the GPU test of the exp path
 * checks the hardware's side.
 * ------------------------------------------------------------------------ */
#define OR_U 5.9604644775390625e-08               /* 2^-24, fp32 unit roundoff */
#define OR_LOG2E 1.44269504088896340736           /* log2 e */
#define OR_LOG2E_F32 1.44269502162933349609375    /* its nearest fp32 value */
#define OR_EXP_HW_ULP 1.0
#define OR_EXP_LIBM_REL (1.01 * OR_U)             /* glibc's expf: < 0.51 ulp */

static double or_band_scale = 1.0; /* test knob: the flags' bands times this (1 = the derived band) */
static int or_exp_perturb = 0;     /* test knob: 0 off; +1 / -1 every G moved to an edge of its
                                    * band; 2 the edge chosen per power */

double or_exp_band(float p)
{
    const double dy = fabs((double)p) * (fabs(OR_LOG2E_F32 - OR_LOG2E) + OR_LOG2E_F32 * OR_U);
    const double e_arg = exp2(dy) - 1.0;
    return (1.0 + e_arg) * (1.0 + OR_EXP_HW_ULP * 2.0 * OR_U) / (1.0 - OR_EXP_LIBM_REL) - 1.0;
}

double or_alpha_band(float p)
{
    return ((1.0 + or_exp_band(p)) * (1.0 + OR_U) / (1.0 - OR_U) - 1.0) * or_band_scale;
}

double or_exp_libm_rel(void) { return OR_EXP_LIBM_REL; }
double or_exp_hw_ulp(void) { return OR_EXP_HW_ULP; }
void or_set_band_scale(double s) { or_band_scale = s; }
void or_set_exp_perturb(int mode) { or_exp_perturb = mode; }

/* A G the GPU could return where this oracle returns G: G moved towards an
 * edge of its band (a little inside it, so that the rounding to fp32 stays
 * within it). */
static float or_perturbed_exp(float p, float G)
{
    double s = (double)or_exp_perturb;
    if (or_exp_perturb == 2) {
        uint32_t b;
        memcpy(&b, &p, 4);
        b = (b ^ (b >> 13)) * 0x9e3779b1u;
        s = ((b >> 17) & 1u) ? 1.0 : -1.0;
    }
    return (float)((double)G * (1.0 + s * (or_exp_band(p) - 1.01 * OR_U)));
}

/* expf and the band, element-wise (for the tests of the band). */
void or_expf_batch(const float* p, float* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = expf(p[i]);
}

void or_exp_band_batch(const float* p, double* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = or_exp_band(p[i]);
}

/* ---- fp32 instantiation --------------------------------------------------- */
#define REAL float
#define SFX f32
#define OR_IS_F32 1
#define R_SQRT sqrtf
#define R_FLOOR floorf
#define R_CEIL ceilf
#define R_EXP expf
#define R_FMA fmaf
#define R_FMAX fmaxf
#define R_FMIN fminf
#include "gs_oracle_body.h"
#undef REAL
#undef SFX
#undef OR_IS_F32
#undef R_SQRT
#undef R_FLOOR
#undef R_CEIL
#undef R_EXP
#undef R_FMA
#undef R_FMAX
#undef R_FMIN

/* ---- fp64 instantiation --------------------------------------------------- */
#define REAL double
#define SFX f64
#define OR_IS_F32 0
#define R_SQRT sqrt
#define R_FLOOR floor
#define R_CEIL ceil
#define R_EXP exp
#define R_FMA fma
#define R_FMAX fmax
#define R_FMIN fmin
#include "gs_oracle_body.h"

/* ---------------------------------------------------------------------------
 * Intersection keys, the plain definition: for each visible (view v, Gaussian
 * g) and each tile tau of its rectangle, key = ((v * T + tau) << 32) | bits(z)
 * with bits() the IEEE-754 pattern of the fp32 view-space depth (monotone for
 * z > 0), payload g; sorted ascending by (key, g), which is a total order
 * because each (v, tau, g) occurs once.
 * rect [V][n][4] = x0 y0 x1 y1 (tiles), visible [V][n], z [V][n] fp32.
 * Returns K (keys written only when K <= capacity).
 * ------------------------------------------------------------------------ */
typedef struct {
    uint64_t key;
    uint32_t val;
} or_kv;

static int cmp_kv(const void* pa, const void* pb)
{
    const or_kv* a = (const or_kv*)pa;
    const or_kv* b = (const or_kv*)pb;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    return (a->val > b->val) - (a->val < b->val);
}

int64_t or_emit_sorted(const int32_t* rect, const uint8_t* visible, const float* z, int64_t n, int V,
                       int TX, int TY, uint64_t* keys, uint32_t* vals, int64_t capacity)
{
    const int64_t T = (int64_t)TX * TY;
    int64_t K = 0;
    for (int64_t i = 0; i < (int64_t)V * n; ++i) {
        if (!visible[i]) continue;
        const int32_t* r = rect + 4 * i;
        K += (int64_t)(r[2] - r[0]) * (r[3] - r[1]);
    }
    if (K > capacity) return K;
    or_kv* kv = (or_kv*)malloc(sizeof(or_kv) * (size_t)(K > 0 ? K : 1));
    int64_t k = 0;
    for (int v = 0; v < V; ++v)
        for (int64_t g = 0; g < n; ++g) {
            const int64_t i = (int64_t)v * n + g;
            if (!visible[i]) continue;
            const int32_t* r = rect + 4 * i;
            uint32_t zb;
            memcpy(&zb, &z[i], 4);
            for (int ty = r[1]; ty < r[3]; ++ty)
                for (int tx = r[0]; tx < r[2]; ++tx) {
                    const uint64_t tile = (uint64_t)v * (uint64_t)T + (uint64_t)ty * TX + tx;
                    kv[k].key = (tile << 32) | zb;
                    kv[k].val = (uint32_t)g;
                    ++k;
                }
        }
    qsort(kv, (size_t)K, sizeof(or_kv), cmp_kv);
    for (int64_t i = 0; i < K; ++i) {
        keys[i] = kv[i].key;
        vals[i] = kv[i].val;
    }
    free(kv);
    return K;
}

/* ranges [n_tiles_total][2]: first index and one past the last index of each
 * tile id (key >> 32) in the sorted list; (0, 0) for a tile with no entry. */
void or_tile_ranges(const uint64_t* keys, int64_t K, int64_t n_tiles_total, uint32_t* ranges)
{
    for (int64_t t = 0; t < 2 * n_tiles_total; ++t) ranges[t] = 0;
    for (int64_t i = 0; i < K; ++i) {
        const uint64_t t = keys[i] >> 32;
        if (i == 0 || (keys[i - 1] >> 32) != t) ranges[2 * t] = (uint32_t)i;
        if (i == K - 1 || (keys[i + 1] >> 32) != t) ranges[2 * t + 1] = (uint32_t)(i + 1);
    }
}

/* out[i] = sum_{j<i} in[j], out[count] = total. */
void or_exclusive_scan(const uint32_t* in, int64_t count, uint64_t* out)
{
    uint64_t s = 0;
    for (int64_t i = 0; i < count; ++i) {
        out[i] = s;
        s += in[i];
    }
    out[count] = s;
}

/* Adam, Kingma & Ba Algorithm 1, step t (1-based), computed in fp64 from the
 * fp32 state and stored back in fp32:
 *   m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *   theta <- theta - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) */
void or_adam(float* theta, const float* g, float* m, float* v, int64_t count, double lr, double b1,
             double b2, double eps, int64_t t)
{
    const double bc1 = 1.0 - pow(b1, (double)t);
    const double bc2 = 1.0 - pow(b2, (double)t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double gi = g[i];
        const double mi = b1 * (double)m[i] + (1.0 - b1) * gi;
        const double vi = b2 * (double)v[i] + (1.0 - b2) * gi * gi;
        const double th = (double)theta[i] - lr * (mi / bc1) / (sqrt(vi / bc2) + eps);
        m[i] = (float)mi;
        v[i] = (float)vi;
        theta[i] = (float)th;
    }
}
