// gs_rasterize_bwd: back-to-front gradients of the alpha compositing to the
// 2D quantities of every (view, Gaussian) (backward rasterization of the
// ByteSplat abstract), on the work decomposition of raster_fwd.hip: one
// wavefront per 8x8 quarter of a tile, each 16-lane DPP row owning a 4x4
// sub-block with its own list of entries.
//
// For I = sum_i c_i a_i T_i + T_final bg over the blended entries of a pixel
// (T_i = prod_{j<i} (1 - a_j), a = min(0.99, o G), G = exp(power)):
//   dI/dc_i = a_i T_i
//   dI/da_i = T_i (c_i - S_i), S_i the colour behind entry i normalised by
//             T_{i+1}: S <- a_i c_i + (1 - a_i) S walking back from S = bg
//   da/do = G and da/dpower = o G unless the 0.99 clamp is active
//   dpower/du = -(A dx + B dy), dpower/dv = -(B dx + C dy),
//   dpower/dA = -dx^2/2, dpower/dB = -dx dy, dpower/dC = -dy^2/2.
//
// Only dL/dI . S is needed, never S itself: each lane keeps that one scalar
// (sum over channels of dL/dI_c S_c, with the same recurrence) instead of the
// three channels.
//
// Each row works through its entries in sub-batches of 8, in two phases:
//   1. pixel-parallel, entries in reverse order: every lane rebuilds
//      T_i = T_{i+1} / (1 - a_i) and dL/dI . S for its pixel and writes two
//      numbers per (pixel, entry) to LDS: (dL/da_i) G_i (zero when clamped or
//      not blended) and a_i T_i;
//   2. entry-parallel: lane pairs own one entry each and sum the nine
//      gradient terms over 8 of the sub-block's 16 pixels (two rows of four)
//      from those two numbers: the moments of dx, dy, formed from the
//      weights summed per column and per row and the 4 + 2 distinct dx and
//      dy, scaled by o at the end; one DPP step joins the pair, and the pair's first
//      lane adds the nine sums into the wave's LDS table of its entry (rows
//      holding the same entry add into the same sums, one row after the
//      other).
// No cross-lane reduction runs per (pixel, entry). After each batch of 64
// entries every entry with a contribution issues its global fp32 atomics.
//
// A row's list holds byte offsets of the staged records; its tail, up to the
// longest row's count, holds an extra slot of opacity 0, which no pixel
// blends, so phase 1 needs no per-entry bound test.
#include "raster_common.h"

namespace gs {

constexpr int SUB = 8;            // entries per row per sub-batch
constexpr int CSTRIDE = SUB + 1;  // padded slot stride of the coefficient table
constexpr uint32_t SLOT_BYTES = 32;                   // (u v -A/2 -B) (-C/2 o r g) per slot
constexpr uint32_t PAD_OFF = RW_BATCH * SLOT_BYTES;  // the opacity-0 slot

__global__ __launch_bounds__(RW_THREADS) void k_raster_bwd(const float* __restrict__ rec, int64_t n,
                                                           const uint32_t* __restrict__ ranges,
                                                           const uint32_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ masks, int W, int H, int TX,
                                                           int T, int row0, float bg0, float bg1, float bg2,
                                                           const float* __restrict__ T_final,
                                                           const int32_t* __restrict__ n_contrib,
                                                           const float* __restrict__ dL_dimage,
                                                           float* __restrict__ grad2d)
{
#pragma clang fp contract(off)
    // about 10 KB of LDS per wave, so that 16 waves fit a CU
    __shared__ float4 s_rec[2 * (RW_BATCH + 1)];  // (u v -A/2 -B) (-C/2 o r g) per slot, + the padding slot
    __shared__ float s_b[RW_BATCH + 1];           // blue of each slot
    __shared__ uint8_t s_mask[RW_BATCH];
    __shared__ __align__(16) uint16_t s_list[4 * RW_BATCH];  // record byte offsets, read 8 at a time
    __shared__ float s_sum[GS_GRAD2D_ROWS][RW_BATCH];  // [gradient][slot], summed over the rows
    __shared__ float2 s_coef[4][16][CSTRIDE];          // [row][pixel][slot]
    __shared__ uint32_t s_gid[RW_BATCH];               // Gaussian of each staged slot
    __shared__ uint8_t s_live[RW_BATCH];               // slots with a contribution, compacted
    const QuarterCtx t = quarter_ctx(W, H, TX, T, row0);
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
    const int32_t row_last = min(row_max16(my_last), (int32_t)(rg.y - rg.x));
    const int32_t rl0 = __builtin_amdgcn_readlane(row_last, 0), rl1 = __builtin_amdgcn_readlane(row_last, 16);
    const int32_t rl2 = __builtin_amdgcn_readlane(row_last, 32), rl3 = __builtin_amdgcn_readlane(row_last, 48);
    const int32_t wave_last = max(max(rl0, rl1), max(rl2, rl3));
    if (wave_last <= 0) return;
    const int q = t.lane & 15;
    if (t.lane == 0) {  // the padding slot: opacity 0 (alpha 0 at every pixel)
        s_rec[2 * RW_BATCH] = make_float4(0.f, 0.f, 0.f, 0.f);
        s_rec[2 * RW_BATCH + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        s_b[RW_BATCH] = 0.f;
    }
    // phase-2 lanes (e, h) sum over pixels h*8 .. h*8+7 of their row: the
    // dL/dimage of those pixels, taken from the lanes that own them
    float gh0[8], gh1[8], gh2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int src = (t.lane & ~15) + (q >> 3) * 8 + k;
        gh0[k] = __shfl(g0, src);
        gh1[k] = __shfl(g1, src);
        gh2[k] = __shfl(g2, src);
    }
    const float* rv = rec + (int64_t)t.view * n * GS_REC_FLOATS;
    float* g2d = grad2d + (int64_t)t.view * n * GS_GRAD2D_ROWS;  // [n][9] records of this view
    // phase 2: pixel centres of the columns of this row's 4x4 sub-block and
    // of the first of the lane's two rows (h = (lane & 15) >> 3)
    const float sbx = (float)(t.qx0 + (t.row & 1) * 4) + 0.5f;
    const float pxc[4] = {sbx, sbx + 1.f, sbx + 2.f, sbx + 3.f};
    const float pyc0 = (float)(t.qy0 + (t.row >> 1) * 4 + 2 * ((t.lane & 15) >> 3)) + 0.5f;
    float2(*coef)[CSTRIDE] = s_coef[t.row];
    // dL/dI . S, S the colour behind the current entry normalised by the
    // transmittance in front of it; S starts as the background
    float sproj = __builtin_fmaf(g2, bg2, __builtin_fmaf(g1, bg1, g0 * bg0));
    const char* recb = (const char*)s_rec;
    const char* bb = (const char*)s_b;
    // lane s of a batch holds list position hi - s (1-based): slots run back
    // to front. Two-stage prefetch as in the forward pass.
    Entry cur, nxt, nx2;
    {
        const int32_t p0 = wave_last - t.lane, p1 = wave_last - RW_BATCH - t.lane;
        load_entry(cur, p0 >= 1, rg.x + (uint32_t)(p0 - 1), vals, masks, t);
        gather_record(cur, rv);
        load_entry(nxt, p1 >= 1, rg.x + (uint32_t)(p1 - 1), vals, masks, t);
    }
    for (int32_t hi = wave_last; hi >= 1; hi -= RW_BATCH) {
        stage_entry_pair(cur, t.lane, s_rec, s_b, s_mask);
#pragma unroll
        for (int k = 0; k < GS_GRAD2D_ROWS; ++k) s_sum[k][t.lane] = 0.f;
        gather_record(nxt, rv);
        const int32_t p2 = hi - 2 * RW_BATCH - t.lane;
        load_entry(nx2, p2 >= 1, rg.x + (uint32_t)(p2 - 1), vals, masks, t);
        // per row, the staged slots in front of the row's last contributor,
        // ascending, as record offsets; the rest of the row's list is padding
        uint32_t cnt[4];
        {
            asm volatile("" ::: "memory");  // staging writes precede these reads (LDS is in order per wave)
            const uint32_t m4 = s_mask[t.lane];
            const int32_t pos = hi - t.lane;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t rl = r == 0 ? rl0 : r == 1 ? rl1 : r == 2 ? rl2 : rl3;
                const bool keep = ((m4 >> r) & 1u) && pos <= rl;
                const uint64_t m = ballot(keep);
                cnt[r] = (uint32_t)__popcll(m);
                if (keep) s_list[r * RW_BATCH + mask_rank(m)] = (uint16_t)(t.lane * SLOT_BYTES);
                if ((uint32_t)t.lane >= cnt[r]) s_list[r * RW_BATCH + t.lane] = (uint16_t)PAD_OFF;
            }
            asm volatile("" ::: "memory");  // list writes precede their reads
        }
        const uint32_t my_cnt = t.row == 0 ? cnt[0] : t.row == 1 ? cnt[1] : t.row == 2 ? cnt[2] : cnt[3];
        const uint32_t iters = max(max(cnt[0], cnt[1]), max(cnt[2], cnt[3]));
        const uint16_t* my_list = s_list + t.row * RW_BATCH;
        // slot k is in front of this pixel's last contributor iff hi - k <= my_last
        const int32_t thr = (hi - my_last) * (int32_t)SLOT_BYTES;
        for (uint32_t sb = 0; sb < iters; sb += SUB) {
            // ---- phase 1: this lane's pixel, entries sb .. sb+7 of its row
            // (their offsets in one 16-byte read)
            const uint32_t n_sub = min((uint32_t)SUB, iters - sb);
            const uint4 ids = *(const uint4*)(my_list + sb);
            const uint32_t idw[4] = {ids.x, ids.y, ids.z, ids.w};
#pragma unroll
            for (uint32_t i = 0; i < (uint32_t)SUB; ++i) {
                if (i >= n_sub) break;  // wave-uniform
                const uint32_t off = (idw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
                const float4 q0 = *(const float4*)(recb + off);
                const float4 q1 = *(const float4*)(recb + off + 16);
                const float qb = *(const float*)(bb + (off >> 3));
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                const float G = exp_fast(power);
                const float oG = q1.y * G;
                const float alpha = fminf(ALPHA_MAX, oG);
                // the forward's decision for this pixel
                const bool contrib = (int32_t)off >= thr && !(power > 0.f) && !(alpha < ALPHA_MIN);
                // transmittance in front of this entry (a reciprocal: the
                // gradients need no correctly rounded division)
                Tr = contrib ? Tr * __builtin_amdgcn_rcpf(1.f - alpha) : Tr;
                const float ak = contrib ? alpha : 0.f;
                // dI/da = T (c - S), projected on dL/dI; then S' = S + a (c - S)
                const float d = __builtin_fmaf(g2, qb, __builtin_fmaf(g1, q1.w, g0 * q1.z)) - sproj;
                const float dLda = Tr * d;
                sproj = __builtin_fmaf(ak, d, sproj);
                const float dG = (contrib && !(oG > ALPHA_MAX)) ? dLda * G : 0.f;
                coef[q][i] = make_float2(dG, ak * Tr);
            }
            asm volatile("" ::: "memory");  // phase-1 writes precede phase-2 reads (in order per wave)
            // ---- phase 2: lanes (e, h) = (q & 7, q >> 3): entry e of the
            // sub-batch, pixels h*8 .. h*8+7 of the sub-block, i.e. offsets
            // (k & 3, 2h + (k >> 2)) from its first pixel centre, k = 0..7
            const uint32_t e = (uint32_t)q & 7u, h = (uint32_t)q >> 3;
            const uint32_t off_e = my_list[sb + e];
            const float4 q0 = *(const float4*)(recb + off_e);
            const float4 q1 = *(const float4*)(recb + off_e + 16);
            // the lane's 8 pixels are columns x = 0..3 of rows y = 0, 1 (of
            // its half of the sub-block): with dx_x = u - (x centre) and dy_y
            // = v - (y centre), each moment is a sum of weight times products
            // of dx_x, dy_y, formed from per-column and per-row weight sums
            // (dx, dy exactly as in a per-pixel sum: no expansion about a
            // far-away origin, whose terms would cancel)
            float cw[8], gr = 0.f, gg = 0.f, gb = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) cw[k] = 0.f;
            if (e < n_sub) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float2 c = coef[(int)h * 8 + k][e];
                    cw[k] = c.x;
                    gr = __builtin_fmaf(c.y, gh0[k], gr);
                    gg = __builtin_fmaf(c.y, gh1[k], gg);
                    gb = __builtin_fmaf(c.y, gh2[k], gb);
                }
            }
            asm volatile("" ::: "memory");  // phase-2 reads precede the next phase-1 writes
            float dxs[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) dxs[x] = q0.x - pxc[x];
            const float dy0 = q0.y - pyc0, dy1 = q0.y - (pyc0 + 1.f);
            float t0 = cw[0] * dxs[0], t1 = cw[4] * dxs[0], r0 = cw[0], r1 = cw[4];
            float mxx = (cw[0] + cw[4]) * (dxs[0] * dxs[0]);
#pragma unroll
            for (int x = 1; x < 4; ++x) {
                t0 = __builtin_fmaf(cw[x], dxs[x], t0);
                t1 = __builtin_fmaf(cw[4 + x], dxs[x], t1);
                r0 += cw[x];
                r1 += cw[4 + x];
                mxx = __builtin_fmaf(cw[x] + cw[4 + x], dxs[x] * dxs[x], mxx);
            }
            float go = r0 + r1;
            float mx = t0 + t1;
            float my = __builtin_fmaf(r0, dy0, r1 * dy1);
            float mxy = __builtin_fmaf(t0, dy0, t1 * dy1);
            float myy = __builtin_fmaf(r0, dy0 * dy0, r1 * (dy1 * dy1));
            // join the two pixel halves of each entry (lanes q and q + 8): row_ror:8
#define GS_ROR8(v) (v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false)))
            go = GS_ROR8(go);
            mx = GS_ROR8(mx);
            my = GS_ROR8(my);
            mxx = GS_ROR8(mxx);
            mxy = GS_ROR8(mxy);
            myy = GS_ROR8(myy);
            gr = GS_ROR8(gr);
            gg = GS_ROR8(gg);
            gb = GS_ROR8(gb);
#undef GS_ROR8
            // dL/dpower = (dL/da) o G: the o factor is applied here
            const float o = q1.y, nA = q0.z, nB = q0.w, nC = q1.x;
            const float Mx = o * mx, My = o * my;
            const float gsum[GS_GRAD2D_ROWS] = {2.f * nA * Mx + nB * My,  // u
                                                nB * Mx + 2.f * nC * My,  // v
                                                -0.5f * o * mxx,          // A
                                                -o * mxy,                 // B
                                                -0.5f * o * myy,          // C
                                                go,                       // opacity
                                                gr, gg, gb};
            // Rows holding the same slot add into one LDS sum, one row at a
            // time (LDS operations of a wave complete in order; within a row
            // the slots are distinct): plain read-add-write, which costs far
            // less here than LDS float atomics
            const bool own = h == 0 && sb + e < my_cnt;
            const int idx = (int)(off_e / SLOT_BYTES);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                if (own && t.row == rr) {
#pragma unroll
                    for (int k = 0; k < GS_GRAD2D_ROWS; ++k) s_sum[k][idx] += gsum[k];
                }
                asm volatile("" ::: "memory");
            }
        }
        asm volatile("" ::: "memory");  // row sums precede the flush reads
        // The wave's sum of each staged entry (over the rows whose list held
        // it: the same test as their compaction) goes to global memory. Nine
        // lanes serve one entry, so each atomic instruction touches one
        // 36-byte record per entry instead of nine scattered words.
        {
            const uint32_t m4 = s_mask[t.lane];
            const int32_t pos = hi - t.lane;
            const uint32_t rows = ((m4 & 1u) && pos <= rl0 ? 1u : 0u) | (((m4 >> 1) & 1u) && pos <= rl1 ? 2u : 0u) |
                                  (((m4 >> 2) & 1u) && pos <= rl2 ? 4u : 0u) | (((m4 >> 3) & 1u) && pos <= rl3 ? 8u : 0u);
            const bool live = cur.valid && rows != 0u;
            const uint64_t lm = ballot(live);
            s_gid[t.lane] = cur.gid;
            if (live) s_live[mask_rank(lm)] = (uint8_t)t.lane;
            asm volatile("" ::: "memory");
            const uint32_t nlive = (uint32_t)__popcll(lm);
            const uint32_t ke = (uint32_t)t.lane / 9u, kk = (uint32_t)t.lane - 9u * ke;
            for (uint32_t c = 0; c < nlive; c += 7) {
                const uint32_t ei = c + ke;
                if (t.lane < 63 && ei < nlive) {
                    const int s = s_live[ei];
                    const float a = s_sum[kk][s];
                    if (a != 0.f) atomicAdd(g2d + (int64_t)s_gid[s] * GS_GRAD2D_ROWS + kk, a);
                }
            }
        }
        asm volatile("" ::: "memory");
        cur = nxt;
        nxt.valid = nx2.valid;
        nxt.gid = nx2.gid;
        nxt.m4 = nx2.m4;
    }
}

}  // namespace gs

using namespace gs;

extern "C" {

gs_status gs_rasterize_bwd(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                           const uint16_t* masks, const gs_camera* cams, int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, const float* T_final,
                           const int32_t* n_contrib, const float* dL_dimage, float* grad2d, int32_t accumulate,
                           void* stream)
{
    RasterArgs a;
    if (!raster_args(rec, n, ranges, vals, masks, cams, n_views, row0, rows, bg, a)) return GS_ERR_INVALID_ARGUMENT;
    if (!T_final || !n_contrib || !dL_dimage || (n > 0 && !grad2d)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate && n > 0) {
        if (fill_u32((uint32_t*)grad2d, (uint64_t)n_views * GS_GRAD2D_ROWS * (uint64_t)n, 0u, s) != hipSuccess)
            return GS_ERR_HIP;
    }
    hipLaunchKernelGGL(k_raster_bwd, dim3((unsigned)a.n_blocks), dim3(RW_THREADS), 0, s, rec, n, ranges, vals,
                       masks, a.dc.width, a.dc.height, a.dc.tiles_x, a.T, a.row0, bg[0], bg[1], bg[2], T_final,
                       n_contrib, dL_dimage, grad2d);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
