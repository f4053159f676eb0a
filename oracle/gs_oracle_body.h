/*
 * TEST INFRASTRUCTURE ONLY -- the CPU oracle of the Gaussian-splatting training
 * step. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product path never does.
 *
 * This file is the precision-generic body. gs_oracle.c includes it twice:
 *   REAL = float  (suffix f32): the parity oracle. Every quantity that decides
 *     an integer (culling, radius, tile rectangle, depth key, alpha skip and
 *     stop rules, colour and alpha clamps) is computed in fp32 in the pinned
 *     evaluation order written out below (no contraction: built with
 *     -ffp-contract=off; fmaf only where the order names it). Gradients are
 *     accumulated in fp64 from the fp32 decisions.
 *   REAL = double (suffix f64): the same definition in fp64, used for central
 *     finite differences of the backward pass.
 *
 * What the method computes. The pages describe the step only in prose: a tile-
 * based differentiable rasterizer of 3D Gaussians (the 3DGS method, reference
 * [10] in the list of "A Scalable PyTorch Abstraction for Multi-GPU Gaussian
 * Splatting"), rendering each image through per-tile depth-sorted lists of
 * Gaussian-to-pixel intersections ("AMD ROCm team open-sources distributed 3D
 * Gaussian Splatting...", section "Distributed training architecture and memory
 * scaling"), over 16x16 pixel blocks ("On Scaling Up 3D Gaussian Splatting
 * Training", answer (1) on pixel block size), with 59 fp32 parameters per
 * Gaussian (same page, answer on the storage requirement) trained by Adam
 * (reference [12]). Every formula below is therefore a reading: the plainest
 * form of EWA splatting consistent with those statements.
 */

#ifndef OR_CAT
#define OR_CAT2(a, b) a##_##b
#define OR_CAT(a, b) OR_CAT2(a, b)
#endif
#define FN(x) OR_CAT(x, SFX)

/* ---------------------------------------------------------------------------
 * Spherical harmonics, real form with the Condon-Shortley sign, ordered
 * k = l^2 + l + m (m = -l..l). Constants from their closed forms in fp64,
 * rounded once to REAL.
 * ------------------------------------------------------------------------ */
typedef struct {
    REAL c0, c1, c2a, c2b, c2c, c3a, c3b, c3c, c3d, c3e;
} FN(or_shc);

static FN(or_shc) FN(sh_consts)(void)
{
    FN(or_shc) k;
    k.c0 = (REAL)(1.0 / (2.0 * sqrt(M_PI)));          /* Y_00 */
    k.c1 = (REAL)sqrt(3.0 / (4.0 * M_PI));            /* l = 1 */
    k.c2a = (REAL)(0.5 * sqrt(15.0 / M_PI));          /* xy, yz, xz */
    k.c2b = (REAL)(0.25 * sqrt(5.0 / M_PI));          /* 2z^2 - x^2 - y^2 */
    k.c2c = (REAL)(0.25 * sqrt(15.0 / M_PI));         /* x^2 - y^2 */
    k.c3a = (REAL)(0.25 * sqrt(35.0 / (2.0 * M_PI))); /* m = +-3 */
    k.c3b = (REAL)(0.5 * sqrt(105.0 / M_PI));         /* xyz */
    k.c3c = (REAL)(0.25 * sqrt(21.0 / (2.0 * M_PI))); /* m = +-1 */
    k.c3d = (REAL)(0.25 * sqrt(7.0 / M_PI));          /* m = 0 */
    k.c3e = (REAL)(0.25 * sqrt(105.0 / M_PI));        /* z(x^2 - y^2) */
    return k;
}

/* Y[0..(d+1)^2) at direction (x, y, z) (unit length), pinned product order. */
static void FN(sh_basis)(const FN(or_shc) * K, int deg, REAL x, REAL y, REAL z, REAL* Y)
{
    Y[0] = K->c0;
    if (deg < 1) return;
    Y[1] = -(K->c1 * y);
    Y[2] = K->c1 * z;
    Y[3] = -(K->c1 * x);
    if (deg < 2) return;
    REAL xx = x * x, yy = y * y, zz = z * z;
    REAL xy = x * y, yz = y * z, xz = x * z;
    Y[4] = K->c2a * xy;
    Y[5] = -(K->c2a * yz);
    Y[6] = K->c2b * ((2.0f * zz - xx) - yy);
    Y[7] = -(K->c2a * xz);
    Y[8] = K->c2c * (xx - yy);
    if (deg < 3) return;
    Y[9] = -(K->c3a * (y * (3.0f * xx - yy)));
    Y[10] = K->c3b * (xy * z);
    Y[11] = -(K->c3c * (y * ((4.0f * zz - xx) - yy)));
    Y[12] = K->c3d * (z * ((2.0f * zz - 3.0f * xx) - 3.0f * yy));
    Y[13] = -(K->c3c * (x * ((4.0f * zz - xx) - yy)));
    Y[14] = K->c3e * (z * (xx - yy));
    Y[15] = -(K->c3a * (x * (xx - 3.0f * yy)));
}

/* ---------------------------------------------------------------------------
 * Projection of one Gaussian into one view.
 *
 * rec[OR_REC] (REAL): u v z a b c A B C o r g b  (a,b,c = dilated 2D covariance,
 *                     A,B,C = its inverse "conic" with B the off-diagonal)
 * iv[OR_INT] (int32): visible radius x0 y0 x1 y1 count flags
 *   flags bit0 / bit1: guard-band clamp of x/z, y/z active
 *   flags bit2..4    : colour channel r/g/b clamped at 0
 * Tile rectangle [x0, x1) x [y0, y1) in 16x16 tiles.
 * ------------------------------------------------------------------------ */
static void FN(project_one)(const REAL* P, int64_t n, int64_t g, int deg,
                            const or_camera* cam, REAL* rec, int32_t* iv)
{
    for (int i = 0; i < OR_REC; ++i) rec[i] = 0;
    for (int i = 0; i < OR_INT; ++i) iv[i] = 0;

    const REAL x = P[0 * n + g], y = P[1 * n + g], z = P[2 * n + g];
    const REAL W0 = cam->R[0], W1 = cam->R[1], W2 = cam->R[2];
    const REAL W3 = cam->R[3], W4 = cam->R[4], W5 = cam->R[5];
    const REAL W6 = cam->R[6], W7 = cam->R[7], W8 = cam->R[8];
    const REAL t0 = cam->t[0], t1 = cam->t[1], t2 = cam->t[2];

    /* world -> camera */
    const REAL xc = ((W0 * x + W1 * y) + W2 * z) + t0;
    const REAL yc = ((W3 * x + W4 * y) + W5 * z) + t1;
    const REAL zc = ((W6 * x + W7 * y) + W8 * z) + t2;
    const REAL nearp = (REAL)cam->near_plane, farp = (REAL)cam->far_plane;
    if (!(zc > nearp && zc < farp)) return;

    /* activations: exp and sigmoid evaluated in fp64, rounded once */
    REAL s[3];
    for (int i = 0; i < 3; ++i) s[i] = (REAL)exp((double)P[(3 + i) * n + g]);
    const REAL o = (REAL)(1.0 / (1.0 + exp(-(double)P[10 * n + g])));

    /* unit quaternion (w, x, y, z) -> rotation */
    REAL qw = P[6 * n + g], qx = P[7 * n + g], qy = P[8 * n + g], qz = P[9 * n + g];
    const REAL qn = R_SQRT(((qw * qw + qx * qx) + qy * qy) + qz * qz);
    if (qn > 0) { qw = qw / qn; qx = qx / qn; qy = qy / qn; qz = qz / qn; }
    else { qw = 1; qx = 0; qy = 0; qz = 0; }
    REAL Rm[9];
    Rm[0] = 1.0f - 2.0f * (qy * qy + qz * qz);
    Rm[1] = 2.0f * (qx * qy - qw * qz);
    Rm[2] = 2.0f * (qx * qz + qw * qy);
    Rm[3] = 2.0f * (qx * qy + qw * qz);
    Rm[4] = 1.0f - 2.0f * (qx * qx + qz * qz);
    Rm[5] = 2.0f * (qy * qz - qw * qx);
    Rm[6] = 2.0f * (qx * qz - qw * qy);
    Rm[7] = 2.0f * (qy * qz + qw * qx);
    Rm[8] = 1.0f - 2.0f * (qx * qx + qy * qy);

    /* Sigma3 = M M^T with M = R diag(s) */
    REAL M[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[3 * i + j] = Rm[3 * i + j] * s[j];
    REAL S3[9];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            S3[3 * i + j] = (M[3 * i] * M[3 * j] + M[3 * i + 1] * M[3 * j + 1]) + M[3 * i + 2] * M[3 * j + 2];

    /* EWA: Jacobian of the perspective map at the mean, with the off-axis
     * guard band 1.3 x half field of view on x/z and y/z */
    const REAL fx = cam->fx, fy = cam->fy;
    const REAL limx = 1.3f * ((0.5f * (REAL)cam->width) / fx);
    const REAL limy = 1.3f * ((0.5f * (REAL)cam->height) / fy);
    REAL txz = xc / zc, tyz = yc / zc;
    int flags = 0;
    if (txz < -limx) { txz = -limx; flags |= 1; }
    else if (txz > limx) { txz = limx; flags |= 1; }
    if (tyz < -limy) { tyz = -limy; flags |= 2; }
    else if (tyz > limy) { tyz = limy; flags |= 2; }
    const REAL tx = txz * zc, ty = tyz * zc;
    const REAL zz = zc * zc;
    const REAL J00 = fx / zc, J02 = -(fx * tx) / zz;
    const REAL J11 = fy / zc, J12 = -(fy * ty) / zz;

    /* T = J W (2x3) */
    REAL T[6];
    T[0] = J00 * W0 + J02 * W6;
    T[1] = J00 * W1 + J02 * W7;
    T[2] = J00 * W2 + J02 * W8;
    T[3] = J11 * W3 + J12 * W6;
    T[4] = J11 * W4 + J12 * W7;
    T[5] = J11 * W5 + J12 * W8;

    /* U = T Sigma3, Sigma2 = U T^T */
    REAL U[6];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 3; ++j)
            U[3 * i + j] = (T[3 * i] * S3[j] + T[3 * i + 1] * S3[3 + j]) + T[3 * i + 2] * S3[6 + j];
    REAL a = (U[0] * T[0] + U[1] * T[1]) + U[2] * T[2];
    const REAL b = (U[0] * T[3] + U[1] * T[4]) + U[2] * T[5];
    REAL c = (U[3] * T[3] + U[4] * T[4]) + U[5] * T[5];
    /* screen-space low-pass filter of EWA splatting: +0.3 px^2 */
    a = a + 0.3f;
    c = c + 0.3f;
    const REAL det = a * c - b * b;
    if (!(det > 0)) return;
    const REAL A = c / det, B = -b / det, C = a / det;

    /* 3-sigma radius from the larger eigenvalue */
    const REAL mid = 0.5f * (a + c);
    const REAL lam = mid + R_SQRT(R_FMAX(mid * mid - det, 0.0f));
    const REAL rad = R_CEIL(3.0f * R_SQRT(lam));

    /* projected mean in pixels */
    const REAL u = (fx * xc) / zc + (REAL)cam->cx;
    const REAL v = (fy * yc) / zc + (REAL)cam->cy;

    /* tiles touched by the square [u - r, u + r] x [v - r, v + r] */
    const int TX = (cam->width + 15) / 16, TY = (cam->height + 15) / 16;
    const REAL fx0 = R_FMIN(R_FMAX(R_FLOOR((u - rad) / 16.0f), 0.0f), (REAL)TX);
    const REAL fx1 = R_FMIN(R_FMAX(R_CEIL((u + rad) / 16.0f), 0.0f), (REAL)TX);
    const REAL fy0 = R_FMIN(R_FMAX(R_FLOOR((v - rad) / 16.0f), 0.0f), (REAL)TY);
    const REAL fy1 = R_FMIN(R_FMAX(R_CEIL((v + rad) / 16.0f), 0.0f), (REAL)TY);
    const int x0 = (int)fx0, x1 = (int)fx1, y0 = (int)fy0, y1 = (int)fy1;
    const int count = (x1 - x0) * (y1 - y0);
    if (count <= 0) return;

    /* view-dependent colour from SH: direction from the camera centre */
    const REAL ccx = -((W0 * t0 + W3 * t1) + W6 * t2);
    const REAL ccy = -((W1 * t0 + W4 * t1) + W7 * t2);
    const REAL ccz = -((W2 * t0 + W5 * t1) + W8 * t2);
    REAL dx = x - ccx, dy = y - ccy, dz = z - ccz;
    const REAL dn = R_SQRT((dx * dx + dy * dy) + dz * dz);
    dx = dx / dn; dy = dy / dn; dz = dz / dn;
    FN(or_shc) K = FN(sh_consts)();
    REAL Y[16];
    FN(sh_basis)(&K, deg, dx, dy, dz, Y);
    const int nb = (deg + 1) * (deg + 1);
    REAL rgb[3];
    for (int ch = 0; ch < 3; ++ch) {
        REAL acc = Y[0] * P[(11 + ch) * n + g];
        for (int k = 1; k < nb; ++k) acc = acc + Y[k] * P[(11 + 3 * k + ch) * n + g];
        acc = acc + 0.5f;
        if (acc < 0) { acc = 0; flags |= 4 << ch; }
        rgb[ch] = acc;
    }

    rec[0] = u; rec[1] = v; rec[2] = zc;
    rec[3] = a; rec[4] = b; rec[5] = c;
    rec[6] = A; rec[7] = B; rec[8] = C;
    rec[9] = o; rec[10] = rgb[0]; rec[11] = rgb[1]; rec[12] = rgb[2];
    iv[0] = 1; iv[1] = (int32_t)rad; iv[2] = x0; iv[3] = y0; iv[4] = x1; iv[5] = y1;
    iv[6] = count; iv[7] = flags;
}

/* Project all Gaussians into all views. rec [V][n][OR_REC], iv [V][n][OR_INT]. */
void FN(or_preprocess)(const REAL* params, int64_t n, int deg, const or_camera* cams, int V,
                       REAL* rec, int32_t* iv)
{
    for (int vw = 0; vw < V; ++vw) {
#pragma omp parallel for schedule(static)
        for (int64_t g = 0; g < n; ++g)
            FN(project_one)(params, n, g, deg, &cams[vw], rec + ((int64_t)vw * n + g) * OR_REC,
                            iv + ((int64_t)vw * n + g) * OR_INT);
    }
}

/* ---------------------------------------------------------------------------
 * Per-tile depth-ordered lists (the definition: every visible Gaussian whose
 * tile rectangle contains the tile, ascending depth, ties by Gaussian index).
 * ------------------------------------------------------------------------ */
typedef struct {
    int64_t* start; /* [T+1] */
    int64_t* ids;   /* [total] */
} FN(or_lists);

static const REAL* FN(g_sort_z);
static int FN(cmp_depth)(const void* pa, const void* pb)
{
    const int64_t ia = *(const int64_t*)pa, ib = *(const int64_t*)pb;
    const REAL za = FN(g_sort_z)[ia * OR_REC + 2], zb = FN(g_sort_z)[ib * OR_REC + 2];
    if (za < zb) return -1;
    if (za > zb) return 1;
    return (ia > ib) - (ia < ib);
}

static FN(or_lists) FN(build_lists)(const REAL* rec, const int32_t* iv, int64_t n, int TX, int TY)
{
    const int64_t T = (int64_t)TX * TY;
    FN(or_lists) L;
    L.start = (int64_t*)calloc((size_t)T + 1, sizeof(int64_t));
    for (int64_t g = 0; g < n; ++g) {
        const int32_t* q = iv + g * OR_INT;
        if (!q[0]) continue;
        for (int ty = q[3]; ty < q[5]; ++ty)
            for (int tx = q[2]; tx < q[4]; ++tx) L.start[(int64_t)ty * TX + tx + 1]++;
    }
    for (int64_t t = 0; t < T; ++t) L.start[t + 1] += L.start[t];
    L.ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L.start[T] > 0 ? L.start[T] : 1));
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    for (int64_t t = 0; t < T; ++t) fill[t] = L.start[t];
    for (int64_t g = 0; g < n; ++g) {
        const int32_t* q = iv + g * OR_INT;
        if (!q[0]) continue;
        for (int ty = q[3]; ty < q[5]; ++ty)
            for (int tx = q[2]; tx < q[4]; ++tx) L.ids[fill[(int64_t)ty * TX + tx]++] = g;
    }
    free(fill);
    /* qsort is not re-entrant with a global; sort tiles serially */
    FN(g_sort_z) = rec;
    for (int64_t t = 0; t < T; ++t)
        qsort(L.ids + L.start[t], (size_t)(L.start[t + 1] - L.start[t]), sizeof(int64_t), FN(cmp_depth));
    return L;
}

static void FN(free_lists)(FN(or_lists) * L)
{
    free(L->start);
    free(L->ids);
}

/* ---------------------------------------------------------------------------
 * Compositing rules of one (pixel, entry) pair, in the pinned order:
 *   dx = u - px, dy = v - py, pixel centre (i + 0.5, j + 0.5)
 *   power = fma(dx, fma(-A/2, dx, -B*dy), (-C/2 * dy) * dy)
 *         = -(A dx^2 + 2 B dx dy + C dy^2) / 2
 *   skip if power > 0
 *   alpha = min(0.99, o * exp(power));  skip if alpha < 1/255
 *   T' = T * (1 - alpha); stop (entry not blended) if T' < 1e-4
 *   w = alpha * T; C_c = fma(rgb_c, w, C_c); T = T'
 * Returns 0 skip, 1 blended, 2 stop.
 *
 * Near-threshold flags (fp32 only), from the band of or_exp_band (the largest
 * difference between a GPU's exp() and this oracle's): bit0 an image-changing
 * decision may go the other way on the GPU, bit1 the 0.99 clamp may (changes
 * only gradients), bit2 the decision was alpha >= 1/255, bit3 it was the stop.
 *   - alpha: the GPU's o G lies in [oG (1 - ra), oG (1 + ra)], ra = or_alpha_band;
 *     a threshold inside that interval is flagged.
 *   - T: *terr bounds |T_gpu / T - 1| for the pixel so far. A blend moves it to
 *     (1 + terr) (1 + a ra / (1 - a)) q^2 - 1 with q = (1 + u) / (1 - u):
 *     1 - alpha differs by at most a ra / (1 - a) before rounding, and
 *     1 - alpha and T (1 - alpha) are each rounded once on each side (2^-24
 *     relative, u) once their operands may differ. A clamped alpha whose whole
 *     interval lies above 0.99 is the same constant on both sides (ra = 0).
 *     The stop T' < 1e-4 is flagged when T' (1 -+ terr') straddles 1e-4.
 * ------------------------------------------------------------------------ */
static inline int FN(pair_eval)(const REAL* r, REAL px, REAL py, REAL Tcur, REAL* alpha_out,
                                REAL* G_out, REAL* Tnext_out, int* amb, double* terr)
{
    const REAL dx = r[0] - px, dy = r[1] - py;
    const REAL nA = -0.5f * r[6], nB = -r[7], nC = -0.5f * r[8];
    const REAL power = R_FMA(dx, R_FMA(nA, dx, nB * dy), (nC * dy) * dy);
    if (power > 0) return 0;
    REAL G = R_EXP(power);
    if (OR_IS_F32 && or_exp_perturb) G = (REAL)or_perturbed_exp((float)power, (float)G);
    const REAL oG = r[9] * G;
    const REAL alpha = R_FMIN((REAL)0.99f, oG);
    double ra = 0;
    if (OR_IS_F32) {
        ra = or_alpha_band((float)power);
        const double lo = (double)oG * (1.0 - ra), hi = (double)oG * (1.0 + ra);
        const double amin = (double)(1.0f / 255.0f), amax = (double)0.99f;
        if (lo < amin && !(hi < amin)) *amb |= 1 | 4;
        if (!(lo > amax) && hi > amax) *amb |= 2;
        if (lo > amax) ra = 0; /* clamped on both sides */
    }
    if (alpha < (REAL)(1.0f / 255.0f)) return 0;
    const REAL Tn = Tcur * (1.0f - alpha);
    if (OR_IS_F32) {
        double e = *terr;
        if (ra > 0 || e > 0) {
            const double a = (double)alpha, q = (1.0 + OR_U) / (1.0 - OR_U);
            e = (1.0 + e) * (1.0 + a * ra / (1.0 - a)) * q * q - 1.0;
        }
        const double tmin = (double)1e-4f;
        if ((double)Tn * (1.0 - e) < tmin && !((double)Tn * (1.0 + e) < tmin)) *amb |= 1 | 8;
        if (!(Tn < (REAL)1e-4f)) *terr = e;
    }
    *alpha_out = alpha;
    *G_out = G;
    *Tnext_out = Tn;
    if (Tn < (REAL)1e-4f) return 2;
    return 1;
}

/* Forward render of all views (all views share one image size).
 * image [V][3][H][W], T_final [V][H][W], n_contrib [V][H][W] (1-based list
 * position of the last blended entry, 0 if none), amb [V][H][W] flags as
 * above, sig [V][H][W] a hash of every decision taken at that pixel. */
void FN(or_render_fwd)(const REAL* rec, const int32_t* iv, int64_t n, const or_camera* cams, int V,
                       const float* bg, REAL* image, REAL* T_final, int32_t* n_contrib,
                       uint8_t* amb, uint64_t* sig)
{
    const int W = cams[0].width, H = cams[0].height;
    const int TX = (W + 15) / 16, TY = (H + 15) / 16;
    const int64_t HW = (int64_t)H * W;
    for (int vw = 0; vw < V; ++vw) {
        const REAL* rv = rec + (int64_t)vw * n * OR_REC;
        FN(or_lists) L = FN(build_lists)(rv, iv + (int64_t)vw * n * OR_INT, n, TX, TY);
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t tile = 0; tile < (int64_t)TX * TY; ++tile) {
            const int tx = (int)(tile % TX), ty = (int)(tile / TX);
            for (int j = ty * 16; j < ty * 16 + 16 && j < H; ++j)
                for (int i = tx * 16; i < tx * 16 + 16 && i < W; ++i) {
                    const REAL px = (REAL)i + 0.5f, py = (REAL)j + 0.5f;
                    REAL T = 1, col[3] = {0, 0, 0};
                    int last = 0, flags = 0;
                    double terr = 0;
                    uint64_t h = 1469598103934665603ull;
                    for (int64_t e = L.start[tile]; e < L.start[tile + 1]; ++e) {
                        const REAL* r = rv + L.ids[e] * OR_REC;
                        REAL al = 0, G = 0, Tn = 0;
                        const int res = FN(pair_eval)(r, px, py, T, &al, &G, &Tn, &flags, &terr);
                        const int clampd = (res != 0) && (r[9] * G > (REAL)0.99f);
                        h = (h ^ (uint64_t)((e - L.start[tile]) * 8 + res * 2 + clampd)) * 1099511628211ull;
                        if (res == 2) break;
                        if (res == 1) {
                            const REAL w = al * T;
                            for (int ch = 0; ch < 3; ++ch) col[ch] = R_FMA(r[10 + ch], w, col[ch]);
                            T = Tn;
                            last = (int)(e - L.start[tile]) + 1;
                        }
                    }
                    const int64_t p = (int64_t)j * W + i;
                    for (int ch = 0; ch < 3; ++ch)
                        image[((int64_t)vw * 3 + ch) * HW + p] = col[ch] + T * (REAL)bg[ch];
                    T_final[(int64_t)vw * HW + p] = T;
                    n_contrib[(int64_t)vw * HW + p] = last;
                    if (amb) amb[(int64_t)vw * HW + p] = (uint8_t)flags;
                    if (sig) sig[(int64_t)vw * HW + p] = h;
                }
        }
        FN(free_lists)(&L);
    }
}

/* L1 loss, views averaged: L = (1/V) sum_v mean_{c,p} |I - I*|.
 * dL/dI = sign(I - I*) / (3 H W V), sign(0) = 0. Returns L. */
double FN(or_loss_l1)(const REAL* img, const REAL* tgt, int64_t per_view, int V, REAL* dL)
{
    const double inv = 1.0 / ((double)per_view * (double)V);
    const REAL scale = (REAL)inv;
    double acc = 0;
    for (int64_t k = 0; k < per_view * V; ++k) {
        const REAL d = img[k] - tgt[k];
        acc += fabs((double)d);
        dL[k] = d > 0 ? scale : (d < 0 ? -scale : (REAL)0);
    }
    return acc * inv;
}

/* ---------------------------------------------------------------------------
 * Backward of compositing, per pixel, from the definition
 *   I = sum_i c_i a_i T_i + T_final bg,  T_i = prod_{j<i} (1 - a_j)
 * over the blended entries, a_i = min(0.99, o_i G_i),
 * G_i = exp(-(A dx^2 + 2 B dx dy + C dy^2)/2):
 *   dI/dc_i = a_i T_i
 *   dI/da_i = c_i T_i - (sum_{k>i} c_k a_k T_k + T_final bg) / (1 - a_i)
 *   da/do = G, da/dpower = o G (zero when the 0.99 clamp is active)
 * grad2d [V][n][9] (fp64, accumulated): du dv dA dB dC do dr dg db.
 * gabs (optional) accumulates, per slot, the absolute values of the terms
 * each contribution is summed from (tolerance floors).
 * ------------------------------------------------------------------------ */
void FN(or_render_bwd)(const REAL* rec, const int32_t* iv, int64_t n, const or_camera* cams, int V,
                       const float* bg, const REAL* dL_dimg, double* grad2d, double* gabs)
{
    const int W = cams[0].width, H = cams[0].height;
    const int TX = (W + 15) / 16, TY = (H + 15) / 16;
    const int64_t HW = (int64_t)H * W;
    for (int vw = 0; vw < V; ++vw) {
        const REAL* rv = rec + (int64_t)vw * n * OR_REC;
        FN(or_lists) L = FN(build_lists)(rv, iv + (int64_t)vw * n * OR_INT, n, TX, TY);
        const int64_t total = L.start[(int64_t)TX * TY];
        /* per list-entry accumulators: deterministic, reduced serially below */
        double* acc = (double*)calloc((size_t)(total > 0 ? total : 1) * 18, sizeof(double));
#pragma omp parallel
        {
            int64_t cap = 256;
            int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * cap);
            double* al = (double*)malloc(sizeof(double) * cap);
            double* Gs = (double*)malloc(sizeof(double) * cap);
            int* cl = (int*)malloc(sizeof(int) * cap);
            double* Ti = (double*)malloc(sizeof(double) * (cap + 1));
            double* suf = (double*)malloc(sizeof(double) * 3 * (cap + 1));
#pragma omp for schedule(dynamic, 4)
            for (int64_t tile = 0; tile < (int64_t)TX * TY; ++tile) {
                const int tx = (int)(tile % TX), ty = (int)(tile / TX);
                const int64_t len = L.start[tile + 1] - L.start[tile];
                if (len + 1 > cap) {
                    cap = len + 1;
                    idx = (int64_t*)realloc(idx, sizeof(int64_t) * cap);
                    al = (double*)realloc(al, sizeof(double) * cap);
                    Gs = (double*)realloc(Gs, sizeof(double) * cap);
                    cl = (int*)realloc(cl, sizeof(int) * cap);
                    Ti = (double*)realloc(Ti, sizeof(double) * (cap + 1));
                    suf = (double*)realloc(suf, sizeof(double) * 3 * (cap + 1));
                }
                for (int j = ty * 16; j < ty * 16 + 16 && j < H; ++j)
                    for (int i = tx * 16; i < tx * 16 + 16 && i < W; ++i) {
                        const int64_t p = (int64_t)j * W + i;
                        const double g3[3] = {(double)dL_dimg[((int64_t)vw * 3 + 0) * HW + p],
                                              (double)dL_dimg[((int64_t)vw * 3 + 1) * HW + p],
                                              (double)dL_dimg[((int64_t)vw * 3 + 2) * HW + p]};
                        if (g3[0] == 0 && g3[1] == 0 && g3[2] == 0) continue;
                        const REAL px = (REAL)i + 0.5f, py = (REAL)j + 0.5f;
                        /* forward decisions in REAL */
                        REAL T = 1;
                        int m = 0, dummy = 0;
                        double terr = 0;
                        for (int64_t e = L.start[tile]; e < L.start[tile + 1]; ++e) {
                            const REAL* r = rv + L.ids[e] * OR_REC;
                            REAL a = 0, G = 0, Tn = 0;
                            const int res = FN(pair_eval)(r, px, py, T, &a, &G, &Tn, &dummy, &terr);
                            if (res == 2) break;
                            if (res == 1) {
                                idx[m] = e;
                                al[m] = (double)a;
                                Gs[m] = (double)G;
                                cl[m] = r[9] * G > (REAL)0.99f;
                                T = Tn;
                                ++m;
                            }
                        }
                        if (m == 0) continue;
                        /* transmittances and colour behind, in fp64 */
                        Ti[0] = 1.0;
                        for (int k = 0; k < m; ++k) Ti[k + 1] = Ti[k] * (1.0 - al[k]);
                        for (int ch = 0; ch < 3; ++ch) suf[3 * m + ch] = Ti[m] * (double)bg[ch];
                        for (int k = m - 1; k >= 0; --k) {
                            const REAL* r = rv + L.ids[idx[k]] * OR_REC;
                            for (int ch = 0; ch < 3; ++ch)
                                suf[3 * k + ch] = suf[3 * (k + 1) + ch] + (double)r[10 + ch] * al[k] * Ti[k];
                        }
                        for (int k = 0; k < m; ++k) {
                            const REAL* r = rv + L.ids[idx[k]] * OR_REC;
                            double* ac = acc + idx[k] * 18;
                            /* dI/da is a sum over channels of differences (own
                             * colour minus colour behind): the tolerance floor
                             * takes the absolute value of every term of it and
                             * of the dpower products, so that cancellation in
                             * any of them is covered whatever the fp32 order */
                            double dIda = 0, dIda_abs = 0;
                            for (int ch = 0; ch < 3; ++ch) {
                                const double c = (double)r[10 + ch];
                                const double dc = g3[ch] * al[k] * Ti[k];
                                ac[6 + ch] += dc;
                                ac[9 + 6 + ch] += fabs(dc);
                                const double t_own = c * Ti[k], t_behind = suf[3 * (k + 1) + ch] / (1.0 - al[k]);
                                dIda += g3[ch] * (t_own - t_behind);
                                dIda_abs += fabs(g3[ch]) * (fabs(t_own) + fabs(t_behind));
                            }
                            if (cl[k]) continue;
                            const double dx = (double)r[0] - (double)px, dy = (double)r[1] - (double)py;
                            const double A = r[6], B = r[7], C = r[8], o = r[9];
                            const double dpow = dIda * o * Gs[k];
                            const double d[6] = {
                                -dpow * (A * dx + B * dy), -dpow * (B * dx + C * dy),
                                -0.5 * dpow * dx * dx, -dpow * dx * dy, -0.5 * dpow * dy * dy,
                                dIda * Gs[k]};
                            const double pa = dIda_abs * o * Gs[k];
                            const double da[6] = {
                                pa * (fabs(A * dx) + fabs(B * dy)), pa * (fabs(B * dx) + fabs(C * dy)),
                                0.5 * pa * dx * dx, pa * fabs(dx * dy), 0.5 * pa * dy * dy, dIda_abs * Gs[k]};
                            for (int q = 0; q < 6; ++q) { ac[q] += d[q]; ac[9 + q] += da[q]; }
                        }
                    }
            }
            free(idx); free(al); free(Gs); free(cl); free(Ti); free(suf);
        }
        for (int64_t e = 0; e < total; ++e) {
            const int64_t g = L.ids[e];
            double* dst = grad2d + ((int64_t)vw * n + g) * 9;
            for (int q = 0; q < 9; ++q) dst[q] += acc[e * 18 + q];
            if (gabs) {
                double* da = gabs + ((int64_t)vw * n + g) * 9;
                for (int q = 0; q < 9; ++q) da[q] += acc[e * 18 + 9 + q];
            }
        }
        free(acc);
        FN(free_lists)(&L);
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the projection to the parameters, summed over views (fp64
 * arithmetic; decisions -- culling, guard-band clamps, colour clamps -- are
 * those of the REAL forward).
 * grad [P][n] (fp64, overwritten; zero where the Gaussian is culled in every
 * view).
 * ------------------------------------------------------------------------ */
static void FN(sh_dbasis)(const FN(or_shc) * Kr, int deg, double x, double y, double z,
                          double* Y, double* dY /* [16][3] */)
{
    const double c0 = Kr->c0, c1 = Kr->c1, c2a = Kr->c2a, c2b = Kr->c2b, c2c = Kr->c2c;
    const double c3a = Kr->c3a, c3b = Kr->c3b, c3c = Kr->c3c, c3d = Kr->c3d, c3e = Kr->c3e;
    for (int k = 0; k < 48; ++k) dY[k] = 0;
    Y[0] = c0;
    if (deg < 1) return;
    Y[1] = -c1 * y; dY[3 * 1 + 1] = -c1;
    Y[2] = c1 * z;  dY[3 * 2 + 2] = c1;
    Y[3] = -c1 * x; dY[3 * 3 + 0] = -c1;
    if (deg < 2) return;
    const double xx = x * x, yy = y * y, zz = z * z;
    Y[4] = c2a * x * y;  dY[12] = c2a * y; dY[13] = c2a * x;
    Y[5] = -c2a * y * z; dY[16] = -c2a * z; dY[17] = -c2a * y;
    Y[6] = c2b * (2 * zz - xx - yy); dY[18] = -2 * c2b * x; dY[19] = -2 * c2b * y; dY[20] = 4 * c2b * z;
    Y[7] = -c2a * x * z; dY[21] = -c2a * z; dY[23] = -c2a * x;
    Y[8] = c2c * (xx - yy); dY[24] = 2 * c2c * x; dY[25] = -2 * c2c * y;
    if (deg < 3) return;
    Y[9] = -c3a * y * (3 * xx - yy);
    dY[27] = -6 * c3a * x * y; dY[28] = -c3a * (3 * xx - 3 * yy);
    Y[10] = c3b * x * y * z;
    dY[30] = c3b * y * z; dY[31] = c3b * x * z; dY[32] = c3b * x * y;
    Y[11] = -c3c * y * (4 * zz - xx - yy);
    dY[33] = 2 * c3c * x * y; dY[34] = -c3c * (4 * zz - xx - 3 * yy); dY[35] = -8 * c3c * y * z;
    Y[12] = c3d * z * (2 * zz - 3 * xx - 3 * yy);
    dY[36] = -6 * c3d * x * z; dY[37] = -6 * c3d * y * z; dY[38] = c3d * (6 * zz - 3 * xx - 3 * yy);
    Y[13] = -c3c * x * (4 * zz - xx - yy);
    dY[39] = -c3c * (4 * zz - 3 * xx - yy); dY[40] = 2 * c3c * x * y; dY[41] = -8 * c3c * x * z;
    Y[14] = c3e * z * (xx - yy);
    dY[42] = 2 * c3e * x * z; dY[43] = -2 * c3e * y * z; dY[44] = c3e * (xx - yy);
    Y[15] = -c3a * x * (xx - 3 * yy);
    dY[45] = -c3a * (3 * xx - 3 * yy); dY[46] = 6 * c3a * x * y;
}

void FN(or_preprocess_bwd)(const REAL* params, int64_t n, int deg, const or_camera* cams, int V,
                           const double* grad2d, double* grad)
{
    const int Prow = 11 + 3 * (deg + 1) * (deg + 1);
    const int nb = (deg + 1) * (deg + 1);
    FN(or_shc) Kr = FN(sh_consts)();
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n; ++g) {
        double G[59];
        for (int r = 0; r < Prow; ++r) G[r] = 0;
        const double x = params[0 * n + g], y = params[1 * n + g], z = params[2 * n + g];
        double s[3];
        for (int i = 0; i < 3; ++i) s[i] = exp((double)params[(3 + i) * n + g]);
        const double o = 1.0 / (1.0 + exp(-(double)params[10 * n + g]));
        const double q0[4] = {params[6 * n + g], params[7 * n + g], params[8 * n + g], params[9 * n + g]};
        double qn = sqrt(q0[0] * q0[0] + q0[1] * q0[1] + q0[2] * q0[2] + q0[3] * q0[3]);
        double q[4];
        const int qzero = !(qn > 0);
        if (!qzero) for (int i = 0; i < 4; ++i) q[i] = q0[i] / qn;
        else { q[0] = 1; q[1] = q[2] = q[3] = 0; qn = 1; }
        const double w = q[0], qx = q[1], qy = q[2], qz = q[3];
        double Rm[9] = {1 - 2 * (qy * qy + qz * qz), 2 * (qx * qy - w * qz), 2 * (qx * qz + w * qy),
                        2 * (qx * qy + w * qz), 1 - 2 * (qx * qx + qz * qz), 2 * (qy * qz - w * qx),
                        2 * (qx * qz - w * qy), 2 * (qy * qz + w * qx), 1 - 2 * (qx * qx + qy * qy)};
        double M[9], S3[9];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) M[3 * i + j] = Rm[3 * i + j] * s[j];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                S3[3 * i + j] = M[3 * i] * M[3 * j] + M[3 * i + 1] * M[3 * j + 1] + M[3 * i + 2] * M[3 * j + 2];

        double gM[9] = {0}, gp[3] = {0}, gop = 0;
        int any = 0;
        for (int vw = 0; vw < V; ++vw) {
            REAL recr[OR_REC];
            int32_t ivr[OR_INT];
            FN(project_one)(params, n, g, deg, &cams[vw], recr, ivr);
            if (!ivr[0]) continue;
            any = 1;
            const double* g2 = grad2d + ((int64_t)vw * n + g) * 9;
            const or_camera* cam = &cams[vw];
            double Wc[9], tc[3];
            for (int i = 0; i < 9; ++i) Wc[i] = cam->R[i];
            for (int i = 0; i < 3; ++i) tc[i] = cam->t[i];
            const double pc[3] = {Wc[0] * x + Wc[1] * y + Wc[2] * z + tc[0],
                                  Wc[3] * x + Wc[4] * y + Wc[5] * z + tc[1],
                                  Wc[6] * x + Wc[7] * y + Wc[8] * z + tc[2]};
            const double fx = cam->fx, fy = cam->fy, zc = pc[2];
            const int clx = ivr[7] & 1, cly = (ivr[7] >> 1) & 1;
            const double limx = 1.3 * (0.5 * cam->width / fx), limy = 1.3 * (0.5 * cam->height / fy);
            double Lx = pc[0] / zc, Ly = pc[1] / zc;
            if (clx) Lx = Lx < 0 ? -limx : limx;
            if (cly) Ly = Ly < 0 ? -limy : limy;
            /* J00 = fx/z, J02 = -fx Lx / z (Lx = clamp(x/z)), J11, J12 likewise */
            const double J00 = fx / zc, J02 = -fx * Lx / zc, J11 = fy / zc, J12 = -fy * Ly / zc;
            double T[6] = {J00 * Wc[0] + J02 * Wc[6], J00 * Wc[1] + J02 * Wc[7], J00 * Wc[2] + J02 * Wc[8],
                           J11 * Wc[3] + J12 * Wc[6], J11 * Wc[4] + J12 * Wc[7], J11 * Wc[5] + J12 * Wc[8]};
            double S2[4] = {0, 0, 0, 0};
            for (int i = 0; i < 2; ++i)
                for (int j = 0; j < 2; ++j) {
                    double acc = 0;
                    for (int k = 0; k < 3; ++k)
                        for (int l = 0; l < 3; ++l) acc += T[3 * i + k] * S3[3 * k + l] * T[3 * j + l];
                    S2[2 * i + j] = acc;
                }
            const double a = S2[0] + 0.3, b = S2[1], c = S2[3] + 0.3;
            const double det = a * c - b * b, d2 = det * det;
            const double gA = g2[2], gB = g2[3], gC = g2[4];
            /* A = c/det, B = -b/det, C = a/det */
            const double ga = gA * (-c * c / d2) + gB * (b * c / d2) + gC * (-b * b / d2);
            const double gb = gA * (2 * b * c / d2) + gB * (-(det + 2 * b * b) / d2) + gC * (2 * a * b / d2);
            const double gc = gA * (-b * b / d2) + gB * (a * b / d2) + gC * (-a * a / d2);
            /* Sigma2 = T S3 T^T: G2 symmetric with off-diagonal gb/2 */
            const double G2[4] = {ga, 0.5 * gb, 0.5 * gb, gc};
            double gS3[9], gT[6];
            for (int k = 0; k < 3; ++k)
                for (int l = 0; l < 3; ++l) {
                    double acc = 0;
                    for (int i = 0; i < 2; ++i)
                        for (int j = 0; j < 2; ++j) acc += T[3 * i + k] * G2[2 * i + j] * T[3 * j + l];
                    gS3[3 * k + l] = acc;
                }
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 3; ++k) {
                    double acc = 0;
                    for (int j = 0; j < 2; ++j)
                        for (int l = 0; l < 3; ++l) acc += G2[2 * i + j] * T[3 * j + l] * S3[3 * l + k];
                    gT[3 * i + k] = 2 * acc;
                }
            /* T = J W: dL/dJ = dL/dT W^T */
            double gJ00 = 0, gJ02 = 0, gJ11 = 0, gJ12 = 0;
            for (int k = 0; k < 3; ++k) {
                gJ00 += gT[k] * Wc[k];
                gJ02 += gT[k] * Wc[6 + k];
                gJ11 += gT[3 + k] * Wc[3 + k];
                gJ12 += gT[3 + k] * Wc[6 + k];
            }
            double gpc[3] = {0, 0, 0};
            /* J -> camera-space mean */
            gpc[2] += gJ00 * (-fx / (zc * zc)) + gJ11 * (-fy / (zc * zc));
            if (clx) gpc[2] += gJ02 * (fx * Lx / (zc * zc));
            else { gpc[0] += gJ02 * (-fx / (zc * zc)); gpc[2] += gJ02 * (2 * fx * pc[0] / (zc * zc * zc)); }
            if (cly) gpc[2] += gJ12 * (fy * Ly / (zc * zc));
            else { gpc[1] += gJ12 * (-fy / (zc * zc)); gpc[2] += gJ12 * (2 * fy * pc[1] / (zc * zc * zc)); }
            /* u = fx x/z + cx, v = fy y/z + cy */
            gpc[0] += g2[0] * fx / zc;
            gpc[1] += g2[1] * fy / zc;
            gpc[2] += -g2[0] * fx * pc[0] / (zc * zc) - g2[1] * fy * pc[1] / (zc * zc);
            for (int i = 0; i < 3; ++i) gp[i] += Wc[i] * gpc[0] + Wc[3 + i] * gpc[1] + Wc[6 + i] * gpc[2];
            /* Sigma3 = M M^T: dL/dM = (G + G^T) M */
            for (int i = 0; i < 3; ++i)
                for (int j = 0; j < 3; ++j) {
                    double acc = 0;
                    for (int k = 0; k < 3; ++k) acc += (gS3[3 * i + k] + gS3[3 * k + i]) * M[3 * k + j];
                    gM[3 * i + j] += acc;
                }
            /* opacity */
            gop += g2[5];
            /* colour */
            const double cc[3] = {-(Wc[0] * tc[0] + Wc[3] * tc[1] + Wc[6] * tc[2]),
                                  -(Wc[1] * tc[0] + Wc[4] * tc[1] + Wc[7] * tc[2]),
                                  -(Wc[2] * tc[0] + Wc[5] * tc[1] + Wc[8] * tc[2])};
            const double e[3] = {x - cc[0], y - cc[1], z - cc[2]};
            const double en = sqrt(e[0] * e[0] + e[1] * e[1] + e[2] * e[2]);
            const double d[3] = {e[0] / en, e[1] / en, e[2] / en};
            double Y[16], dY[48];
            FN(sh_dbasis)(&Kr, deg, d[0], d[1], d[2], Y, dY);
            double gd[3] = {0, 0, 0};
            for (int ch = 0; ch < 3; ++ch) {
                if ((ivr[7] >> (2 + ch)) & 1) continue;
                const double grc = g2[6 + ch];
                for (int k = 0; k < nb; ++k) {
                    const double coef = params[(11 + 3 * k + ch) * n + g];
                    G[11 + 3 * k + ch] += Y[k] * grc;
                    for (int a3 = 0; a3 < 3; ++a3) gd[a3] += grc * coef * dY[3 * k + a3];
                }
            }
            const double ddg = d[0] * gd[0] + d[1] * gd[1] + d[2] * gd[2];
            for (int i = 0; i < 3; ++i) gp[i] += (gd[i] - d[i] * ddg) / en;
        }
        if (any) {
            for (int i = 0; i < 3; ++i) G[i] = gp[i];
            /* M = R diag(s) */
            double gR[9], gs[3] = {0, 0, 0};
            for (int i = 0; i < 3; ++i)
                for (int j = 0; j < 3; ++j) {
                    gR[3 * i + j] = gM[3 * i + j] * s[j];
                    gs[j] += gM[3 * i + j] * Rm[3 * i + j];
                }
            for (int j = 0; j < 3; ++j) G[3 + j] = gs[j] * s[j];
            /* R(q) -> unit quaternion (w, x, y, z) */
            double gq[4];
            gq[0] = gR[1] * (-2 * qz) + gR[2] * (2 * qy) + gR[3] * (2 * qz) + gR[5] * (-2 * qx) +
                    gR[6] * (-2 * qy) + gR[7] * (2 * qx);
            gq[1] = gR[1] * (2 * qy) + gR[2] * (2 * qz) + gR[3] * (2 * qy) + gR[4] * (-4 * qx) +
                    gR[5] * (-2 * w) + gR[6] * (2 * qz) + gR[7] * (2 * w) + gR[8] * (-4 * qx);
            gq[2] = gR[0] * (-4 * qy) + gR[1] * (2 * qx) + gR[2] * (2 * w) + gR[3] * (2 * qx) +
                    gR[5] * (2 * qz) + gR[6] * (-2 * w) + gR[7] * (2 * qz) + gR[8] * (-4 * qy);
            gq[3] = gR[0] * (-4 * qz) + gR[1] * (-2 * w) + gR[2] * (2 * qx) + gR[3] * (2 * w) +
                    gR[4] * (-4 * qz) + gR[5] * (2 * qy) + gR[6] * (2 * qx) + gR[7] * (2 * qy);
            if (!qzero) {
                const double dot = q[0] * gq[0] + q[1] * gq[1] + q[2] * gq[2] + q[3] * gq[3];
                for (int i = 0; i < 4; ++i) G[6 + i] = (gq[i] - q[i] * dot) / qn;
            }
            G[10] = gop * o * (1 - o);
        }
        for (int r = 0; r < Prow; ++r) grad[(int64_t)r * n + g] = G[r];
    }
}

#undef FN
