// The backward walk of one 8x8 quarter: back-to-front gradients of the alpha
// compositing to the 2D quantities of every (view, Gaussian) (backward
// rasterization of the ByteSplat abstract), on the work decomposition of the
// forward walk (raster_fwd.h): one
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
// No cross-lane reduction runs per (pixel, entry). After each batch (up to 64
// entries, compacted as in the forward walk from those that meet the quarter
// and lie in front of the last contributor of a row they meet) every staged
// entry issues its global fp32 atomics.
//
// A row's list holds byte offsets of the staged records; its tail, up to the
// longest row's count, holds an extra slot of opacity 0, which no pixel
// blends, so phase 1 needs no per-entry bound test. Each slot carries its
// list position, which a pixel compares with its own last contributor.
#pragma once

#include "raster_common.h"

namespace gs {

constexpr int BW_SUB = 8;            // entries per row per sub-batch
constexpr int BW_CSTRIDE = BW_SUB + 1;  // padded slot stride of the coefficient table
constexpr uint32_t BW_SLOT_BYTES = 32;                   // (u v -A/2 -B) (-C/2 o r g) per slot
constexpr uint32_t BW_PAD_OFF = RW_BATCH * BW_SLOT_BYTES;  // the opacity-0 slot

// LDS of the backward walk (about 9.8 KB, so that 16 waves fit a CU).
struct BwdLds {
    float4 rec[2 * (RW_BATCH + 1)];            // (u v -A/2 -B) (-C/2 o r g) per slot, + the padding slot
    float2 bp[RW_BATCH + 1];                   // (blue, 1-based list position as int bits) per slot
    alignas(16) uint16_t list[4 * RW_BATCH];   // row lists of record byte offsets (and the batch compaction's scratch)
    float sum[GS_GRAD2D_ROWS][RW_BATCH];       // [gradient][slot], summed over the rows
    float2 coef[4][16][BW_CSTRIDE];            // [row][pixel][slot]
};

// One pixel per lane: my_last its n_contrib (0 outside the image), Tr its
// final transmittance, (g0, g1, g2) its dL/dimage. Adds the quarter's
// gradients into grad2d ([V][n][9]).
__device__ __forceinline__ void raster_bwd_walk(BwdLds& L, const QuarterCtx& t, int32_t my_last, float Tr, float g0,
                                                float g1, float g2, float bg0, float bg1, float bg2,
                                                const float* __restrict__ rec, int64_t n,
                                                const uint32_t* __restrict__ ranges,
                                                const uint32_t* __restrict__ vals,
                                                const uint16_t* __restrict__ masks, uint32_t cap,
                                                float* __restrict__ grad2d)
{
#pragma clang fp contract(off)
    if (g0 == 0.f && g1 == 0.f && g2 == 0.f) my_last = 0;  // this pixel adds nothing
    const uint2 rg = tile_range(ranges, t.tile_lin, cap);
    // never walk past the tile's list, whatever n_contrib holds
    const int32_t row_last = min(row_max16(my_last), (int32_t)(rg.y - rg.x));
    const int32_t rl0 = __builtin_amdgcn_readlane(row_last, 0), rl1 = __builtin_amdgcn_readlane(row_last, 16);
    const int32_t rl2 = __builtin_amdgcn_readlane(row_last, 32), rl3 = __builtin_amdgcn_readlane(row_last, 48);
    const int32_t wave_last = max(max(rl0, rl1), max(rl2, rl3));
    if (wave_last <= 0) return;
    const int q = t.lane & 15;
    if (t.lane == 0) {  // the padding slot: opacity 0 (alpha 0 at every pixel)
        L.rec[2 * RW_BATCH] = make_float4(0.f, 0.f, 0.f, 0.f);
        L.rec[2 * RW_BATCH + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        L.bp[RW_BATCH] = make_float2(0.f, 0.f);
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
    float2(*coef)[BW_CSTRIDE] = L.coef[t.row];
    // dL/dI . S, S the colour behind the current entry normalised by the
    // transmittance in front of it; S starts as the background
    float sproj = __builtin_fmaf(g2, bg2, __builtin_fmaf(g1, bg1, g0 * bg0));
    const char* recb = (const char*)L.rec;
    const char* bpb = (const char*)L.bp;
    // entries back to front, in batches of those that meet the quarter and
    // lie in front of the last contributor of a row they meet (raster_common.h);
    // three batches in flight as in the forward walk
    const int32_t rl[4] = {rl0, rl1, rl2, rl3};
    ChunkScan S = scan_start<true>(wave_last - 1, wave_last, rg.x, masks, t, rl);
    Entry cur, nxt, nx2;
    uint32_t n_cur = take_batch<true>(S, cur, wave_last, rg.x, vals, masks, t, rl, L.list);
    gather_record(cur, rv, n);
    uint32_t n_nxt = take_batch<true>(S, nxt, wave_last, rg.x, vals, masks, t, rl, L.list);
    while (n_cur > 0u || n_nxt > 0u || scan_left<true>(S, wave_last)) {
        stage_entry_pair(cur, t.lane, L.rec, L.bp);
#pragma unroll
        for (int k = 0; k < GS_GRAD2D_ROWS; ++k) L.sum[k][t.lane] = 0.f;
        gather_record(nxt, rv, n);
        const uint32_t n_nx2 = take_batch<true>(S, nx2, wave_last, rg.x, vals, masks, t, rl, L.list);
        // per row, its staged slots (in descending list order), as record
        // offsets; the rest of the row's list is padding
        uint32_t cnt[4];
        {
            asm volatile("" ::: "memory");  // compaction reads precede these writes (LDS is in order per wave)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = (cur.m4 >> r) & 1u;
                const uint64_t m = ballot(keep);
                cnt[r] = (uint32_t)__popcll(m);
                if (keep) L.list[r * RW_BATCH + mask_rank(m)] = (uint16_t)(t.lane * BW_SLOT_BYTES);
                if ((uint32_t)t.lane >= cnt[r]) L.list[r * RW_BATCH + t.lane] = (uint16_t)BW_PAD_OFF;
            }
            asm volatile("" ::: "memory");  // list writes precede their reads
        }
        const uint32_t my_cnt = t.row == 0 ? cnt[0] : t.row == 1 ? cnt[1] : t.row == 2 ? cnt[2] : cnt[3];
        const uint32_t iters = max(max(cnt[0], cnt[1]), max(cnt[2], cnt[3]));
        const uint16_t* my_list = L.list + t.row * RW_BATCH;
        for (uint32_t sb = 0; sb < iters; sb += BW_SUB) {
            // ---- phase 1: this lane's pixel, entries sb .. sb+7 of its row
            // (their offsets in one 16-byte read)
            const uint32_t n_sub = min((uint32_t)BW_SUB, iters - sb);
            const uint4 ids = *(const uint4*)(my_list + sb);
            const uint32_t idw[4] = {ids.x, ids.y, ids.z, ids.w};
#pragma unroll
            for (uint32_t i = 0; i < (uint32_t)BW_SUB; ++i) {
                if (i >= n_sub) break;  // wave-uniform
                const uint32_t off = (idw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
                const float4 q0 = *(const float4*)(recb + off);
                const float4 q1 = *(const float4*)(recb + off + 16);
                const float2 qbp = *(const float2*)(bpb + (off >> 2));  // (blue, list position)
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                const float G = exp_fast(power);
                const float oG = q1.y * G;
                const float alpha = fminf(ALPHA_MAX, oG);
                // the forward's decision for this pixel
                const bool contrib = __float_as_int(qbp.y) <= my_last && !(power > 0.f) && !(alpha < ALPHA_MIN);
                // transmittance in front of this entry (a reciprocal: the
                // gradients need no correctly rounded division)
                Tr = contrib ? Tr * __builtin_amdgcn_rcpf(1.f - alpha) : Tr;
                const float ak = contrib ? alpha : 0.f;
                // dI/da = T (c - S), projected on dL/dI; then S' = S + a (c - S)
                const float d = __builtin_fmaf(g2, qbp.x, __builtin_fmaf(g1, q1.w, g0 * q1.z)) - sproj;
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
            const int idx = (int)(off_e / BW_SLOT_BYTES);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                if (own && t.row == rr) {
#pragma unroll
                    for (int k = 0; k < GS_GRAD2D_ROWS; ++k) L.sum[k][idx] += gsum[k];
                }
                asm volatile("" ::: "memory");
            }
        }
        asm volatile("" ::: "memory");  // row sums precede the flush reads
        // The wave's sum of each staged entry (every slot of the batch holds
        // an entry some row kept) goes to global memory. Nine lanes serve one
        // entry, so each atomic instruction touches one 36-byte record per
        // entry instead of nine scattered words.
        {
            const uint32_t ke = (uint32_t)t.lane / 9u, kk = (uint32_t)t.lane - 9u * ke;
            for (uint32_t c = 0; c < n_cur; c += 7) {
                const uint32_t ei = c + ke;
                const uint32_t g = (uint32_t)__shfl((int)cur.gid, (int)min(ei, 63u));
                if (t.lane < 63 && ei < n_cur && (int64_t)g < n) {
                    const float a = L.sum[kk][ei];
                    if (a != 0.f) atomicAdd(g2d + (int64_t)g * GS_GRAD2D_ROWS + kk, a);
                }
            }
        }
        asm volatile("" ::: "memory");
        cur = nxt;
        nxt.valid = nx2.valid;
        nxt.gid = nx2.gid;
        nxt.m4 = nx2.m4;
        nxt.rel = nx2.rel;
        n_cur = n_nxt;
        n_nxt = n_nx2;
    }
}

}  // namespace gs
