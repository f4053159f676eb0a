// The forward walk of one 8x8 quarter over its tile's sorted list (forward
// rasterization of the ByteSplat abstract; 16x16 pixel blocks of "On Scaling
// Up 3D Gaussian Splatting Training", answer (1); depth-sorted per-tile lists
// of the ROCm page, section "Distributed training architecture and memory
// scaling"). Used by the forward kernels and by the fused forward + loss +
// backward kernel.
//
// Work decomposition (gfx950, wave64):
//   * one 64-lane workgroup per 8x8 quarter of a 16x16 tile, one lane per
//     pixel; the four quarters of a tile are independent wavefronts, so each
//     stops as soon as its own pixels are saturated and nothing waits at a
//     barrier;
//   * each 16-lane DPP row owns a 4x4 sub-block of the quarter and walks its
//     own list of entries;
//   * the tile's sorted list is read in batches of up to 64 entries whose
//     sub-block masks meet the quarter (compacted from up to four chunks of
//     64 list positions, raster_common.h): each lane gathers one entry's
//     48-byte record (the next batch's gathers are in flight while the
//     current batch is evaluated) and stages it in LDS; each row compacts the
//     entries of its sub-block (ballot + mbcnt, list order kept);
//   * in the pixel loop every row reads its own next entry (an LDS broadcast
//     within the row), so one instruction stream advances four sub-blocks on
//     four different entries. An entry skipped by the mask has alpha < 1/255
//     at every pixel of the sub-block and would have been skipped anyway:
//     results are unchanged. Row lists hold record byte offsets and are
//     padded to the longest row's count with a slot of opacity 0 (never
//     blended), so the loop needs no per-entry bound test; each staged
//     record carries its list position for n_contrib.
//
// Per (pixel, entry), in this fixed fp32 order:
//   dx = u - px, dy = v - py
//   power = fma(dx, fma(-A/2, dx, -B*dy), (-C/2*dy)*dy)
//   skip if power > 0; alpha = min(0.99, o * exp(power)); skip if alpha < 1/255
//   T' = T (1 - alpha); stop before this entry if T' < 1e-4
//   w = alpha T; C_c = fma(rgb_c, w, C_c); T = T'
#pragma once

#include "raster_common.h"

namespace gs {

// LDS of the forward walk (about 3.6 KB): records at a stride of 48 bytes and
// an extra slot of opacity 0 that pads each row's list to the longest row's
// count (no pixel blends it), and per row the record byte offsets of its
// entries (read 8 at a time); the row lists double as the scratch of the
// batch compaction, which runs before they are built.
struct FwdLds {
    float4 rec[3 * (RW_BATCH + 1)];
    alignas(16) uint16_t list[4 * RW_BATCH];
};

// What the walk leaves per pixel: transmittance, accumulated colour (without
// the background) and the 1-based list position of the last blended entry.
struct FwdPixel {
    float Tr, C0, C1, C2;
    int32_t last;
};

__device__ __forceinline__ FwdPixel raster_fwd_walk(FwdLds& L, const QuarterCtx& t, const float* __restrict__ rec,
                                                    int64_t n, const uint32_t* __restrict__ ranges,
                                                    const uint32_t* __restrict__ vals,
                                                    const uint16_t* __restrict__ masks, uint32_t cap)
{
#pragma clang fp contract(off)
    constexpr uint32_t SLOT_BYTES = 48, PAD_OFF = RW_BATCH * SLOT_BYTES;
    const uint2 rg = tile_range(ranges, t.tile_lin, cap);
    const float* rv = rec + (int64_t)t.view * n * GS_REC_FLOATS;
    float Tr = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    int32_t last = 0;
    bool done = !t.inside;
    if (t.lane == 0) {
        L.rec[3 * RW_BATCH] = make_float4(0.f, 0.f, 0.f, 0.f);
        L.rec[3 * RW_BATCH + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        L.rec[3 * RW_BATCH + 2] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const char* recb = (const char*)L.rec;
    const int32_t len = (int32_t)(rg.y - rg.x);
    // three batches in flight: records of the next one and ids of the one
    // after are requested while the current one is evaluated
    ChunkScan S = scan_start<false>(0, len, rg.x, masks, t, nullptr);
    Entry cur, nxt, nx2;
    uint32_t n_cur = take_batch<false>(S, cur, len, rg.x, vals, masks, t, nullptr, L.list);
    gather_record(cur, rv, n);
    uint32_t n_nxt = take_batch<false>(S, nxt, len, rg.x, vals, masks, t, nullptr, L.list);
    while (n_cur > 0u || n_nxt > 0u || scan_left<false>(S, len)) {
        if (ballot(!done) == 0ull) break;
        stage_entry(cur, t.lane, L.rec);
        gather_record(nxt, rv, n);
        const uint32_t n_nx2 = take_batch<false>(S, nx2, len, rg.x, vals, masks, t, nullptr, L.list);
        // per row, the staged entries of its sub-block in list order, as
        // record offsets; the rest of the row's list is the padding slot. A
        // row whose 16 pixels have all stopped gets no entries (they could
        // change nothing), so that it does not set the batch's length.
        uint32_t cnt[4];
        {
            const uint64_t live = ballot(!done);
            asm volatile("" ::: "memory");  // compaction reads precede these writes (LDS is in order per wave)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = ((cur.m4 >> r) & 1u) && ((live >> (16 * r)) & 0xffffull) != 0ull;
                const uint64_t m = ballot(keep);
                cnt[r] = (uint32_t)__popcll(m);
                if (keep) L.list[r * RW_BATCH + mask_rank(m)] = (uint16_t)(t.lane * SLOT_BYTES);
                if ((uint32_t)t.lane >= cnt[r]) L.list[r * RW_BATCH + t.lane] = (uint16_t)PAD_OFF;
            }
            asm volatile("" ::: "memory");  // list writes precede their reads
        }
        const uint32_t iters = max(max(cnt[0], cnt[1]), max(cnt[2], cnt[3]));
        const uint16_t* my_list = L.list + t.row * RW_BATCH;
        // groups of 8 entries: their record offsets in one 16-byte read; a
        // full group runs as one straight block (no test between entries),
        // so the scheduler may overlap one entry's LDS reads with the last
        for (uint32_t sb = 0; sb < iters; sb += 8) {
            const uint4 ids = *(const uint4*)(my_list + sb);
            const uint32_t idw[4] = {ids.x, ids.y, ids.z, ids.w};
            auto f1 = [&](uint32_t i) {
                const uint32_t off = (idw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
                const float4 q0 = *(const float4*)(recb + off);
                const float4 q1 = *(const float4*)(recb + off + 16);
                const float2 q2 = *(const float2*)(recb + off + 32);
                // branch-free update: only lanes that blend change state (a
                // zero weight adds exactly 0)
                float dx, dy;
                const float power = entry_power(q0, q1, t.px, t.py, dx, dy);
                const float alpha = fminf(ALPHA_MAX, q1.y * exp_fast(power));
                const float Tn = Tr * (1.f - alpha);
                const bool keep = !done && !(power > 0.f) && !(alpha < ALPHA_MIN);
                const bool stop = keep && Tn < T_MIN;
                const bool blend = keep && !stop;
                const float w = blend ? alpha * Tr : 0.f;
                C0 = __builtin_fmaf(q1.z, w, C0);
                C1 = __builtin_fmaf(q1.w, w, C1);
                C2 = __builtin_fmaf(q2.x, w, C2);
                Tr = blend ? Tn : Tr;
                last = blend ? __float_as_int(q2.y) : last;
                done = done || stop;
            };
            if (sb + 8u <= iters) {
#pragma unroll
                for (uint32_t i = 0; i < 8u; ++i) f1(i);
            } else {
#pragma unroll
                for (uint32_t i = 0; i < 8u; ++i) {
                    if (sb + i >= iters) break;  // wave-uniform
                    f1(i);
                }
            }
            if (ballot(!done) == 0ull) break;
        }
        asm volatile("" ::: "memory");  // this batch's LDS reads precede the next staging
        cur = nxt;
        nxt.valid = nx2.valid;
        nxt.gid = nx2.gid;
        nxt.m4 = nx2.m4;
        nxt.rel = nx2.rel;
        n_cur = n_nxt;
        n_nxt = n_nx2;
    }
    FwdPixel P;
    P.Tr = Tr;
    P.C0 = C0;
    P.C1 = C1;
    P.C2 = C2;
    P.last = last;
    return P;
}

// dL/dI of one channel for L1: scale * sign(I - I*), sign(0) = 0.
__device__ __forceinline__ float l1_grad(float d, float scale) { return d > 0.f ? scale : (d < 0.f ? -scale : 0.f); }

// After the per-quarter partial sums in a raster pass's workspace: the loss
// reduction's per-workgroup sums and its arrival counter. The pass's first
// workgroup resets the counter (so a fresh workspace needs no clearing) and
// the reduction's last workgroup resets it again.
constexpr int LOSS_BLOCKS = 256;
constexpr size_t LOSS_TAIL_BYTES = (LOSS_BLOCKS + 2) * sizeof(double);
__host__ __device__ inline uint32_t* loss_counter(double* partial, int64_t n_partials)
{
    return (uint32_t*)(partial + n_partials + LOSS_BLOCKS);
}

// The wave's sum of `ad` (fp64) written to partial[blockIdx.x] by lane 0.
__device__ __forceinline__ void loss_partial(float ad, int lane, double* __restrict__ partial)
{
    double acc = (double)ad;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) partial[blockIdx.x] = acc;
}

}  // namespace gs
