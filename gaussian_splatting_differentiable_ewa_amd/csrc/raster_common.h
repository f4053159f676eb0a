// Shared pieces of the forward and backward raster kernels: the work unit
// (one wavefront per 8x8 quarter of a 16x16 tile), staging of list entries,
// per-row compaction and the fixed-order per-pair arithmetic. The design is
// described in raster_fwd.hip.
#pragma once

#include "internal.h"

namespace gs {

constexpr int RW_THREADS = 64;  // one wavefront: an 8x8 quarter of a tile
constexpr int RW_BATCH = 64;    // list entries staged per round, one per lane
constexpr float ALPHA_MIN = 1.0f / 255.0f;
constexpr float ALPHA_MAX = 0.99f;
constexpr float T_MIN = 1e-4f;
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

// Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Renumber so that each XCD receives runs of 16 consecutive logical blocks
// (four neighbouring tiles, whose quarters share list entries and records in
// that XCD's L2) while the runs alternate between XCDs (dense and sparse image
// regions spread over all of them).
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t bid, uint32_t nblocks)
{
    constexpr uint32_t CH = 16u;
    const uint32_t full = nblocks / (8u * CH) * (8u * CH);
    if (bid >= full) return bid;
    const uint32_t x = bid & 7u, idx = bid >> 3;
    return (x + 8u * (idx / CH)) * CH + idx % CH;
}

struct QuarterCtx {
    uint32_t view, tile_lin;  // tile_lin = view * tiles_per_view + tile
    int qx0, qy0;             // quarter origin (pixels)
    int mshift;               // bit of the quarter's first sub-block in a 16-bit tile mask
    int lane, row;            // row = 16-lane DPP row = 4x4 sub-block (row & 1, row >> 1)
    int i, j;                 // this lane's pixel: (lane & 3, (lane >> 2) & 3) within the sub-block
    bool inside;
    bool empty;               // the quarter lies outside the image
    float px, py;
};

__device__ __forceinline__ QuarterCtx quarter_ctx(int W, int H, int TX, int T)
{
    QuarterCtx t;
    const uint32_t lb = xcd_chunked(blockIdx.x, gridDim.x);
    const uint32_t quad = lb & 3u;
    t.tile_lin = lb >> 2;
    t.view = t.tile_lin / (uint32_t)T;
    const uint32_t tile = t.tile_lin - t.view * (uint32_t)T;
    const uint32_t ty = tile / (uint32_t)TX, tx = tile - ty * (uint32_t)TX;
    t.qx0 = (int)tx * 16 + (int)(quad & 1u) * 8;
    t.qy0 = (int)ty * 16 + (int)(quad >> 1) * 8;
    t.mshift = (int)(quad >> 1) * 8 + (int)(quad & 1u) * 2;
    t.lane = (int)threadIdx.x;
    t.row = t.lane >> 4;
    const int q = t.lane & 15;
    t.i = t.qx0 + (t.row & 1) * 4 + (q & 3);
    t.j = t.qy0 + (t.row >> 1) * 4 + (q >> 2);
    t.inside = t.i < W && t.j < H;
    t.empty = t.qx0 >= W || t.qy0 >= H;
    t.px = (float)t.i + 0.5f;
    t.py = (float)t.j + 0.5f;
    return t;
}

// One list entry on its way from global memory to LDS. An entry is valid
// when it lies in the list and its sub-block mask meets this quarter; only
// valid entries are gathered.
struct Entry {
    float4 a, b, c;  // record: (u v A B) (C o r g) (b ex ey z)
    uint32_t gid;
    uint32_t m4;     // the quarter's 4 bits of the entry's tile mask
    bool valid;
};

// The quarter's 4 sub-block bits (row r = sub-block (r & 1, r >> 1)) of a
// 16-bit tile mask (bit 4 sy + sx for sub-block (sx, sy) of the tile).
__device__ __forceinline__ uint32_t quarter_bits(uint32_t m16, const QuarterCtx& t)
{
    const uint32_t m = m16 >> t.mshift;
    return (m & 3u) | ((m >> 2) & 0xcu);
}

// Id and mask of list position p (when in the list), for this quarter.
__device__ __forceinline__ void load_entry(Entry& E, bool in_list, uint32_t p, const uint32_t* __restrict__ vals,
                                           const uint16_t* __restrict__ masks, const QuarterCtx& t)
{
    E.m4 = in_list ? quarter_bits(masks[p], t) : 0u;
    E.valid = E.m4 != 0u;
    E.gid = E.valid ? vals[p] : 0u;
}

// An invalid entry gets a zero record (opacity 0): a kernel may evaluate a
// staged slot that no row holds, and must find finite values there.
__device__ __forceinline__ void gather_record(Entry& E, const float* __restrict__ rv)
{
    if (E.valid) {
        const float4* rp = (const float4*)(rv + (int64_t)E.gid * GS_REC_FLOATS);
        E.a = rp[0];
        E.b = rp[1];
        E.c = rp[2];
    } else {
        E.a = E.b = E.c = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Stage the lane's entry at slot `s`: (u, v, -A/2, -B) (-C/2, o, r, g)
// (b, -, -, -), and its 4 sub-block bits for this quarter (0 if invalid).
__device__ __forceinline__ void stage_entry(const Entry& E, int s, float4* __restrict__ s_rec,
                                            uint8_t* __restrict__ s_mask)
{
    s_rec[3 * s + 0] = make_float4(E.a.x, E.a.y, -0.5f * E.a.z, -E.a.w);
    s_rec[3 * s + 1] = make_float4(-0.5f * E.b.x, E.b.y, E.b.z, E.b.w);
    s_rec[3 * s + 2] = make_float4(E.c.x, 0.f, 0.f, 0.f);
    s_mask[s] = (uint8_t)(E.valid ? E.m4 : 0u);
}

// Smallest value of Q(X, y) = A X^2 + 2 B X y + C y^2 over y in [y0, y1]
// (C > 0, rC ~ 1/C); `mag` receives the sum of the magnitudes of its terms.
// An approximate minimiser only raises the value by C times its error
// squared, far below the widening of the test that uses it.
__device__ __forceinline__ float conic_edge_min(float X, float y0, float y1, float A, float B, float C, float rC,
                                                float& mag)
{
    const float ys = fminf(fmaxf(-(B * X) * rC, y0), y1);
    const float t1 = A * X * X, t2 = 2.f * B * X * ys, t3 = C * ys * ys;
    mag = fabsf(t1) + fabsf(t2) + t3;
    return (t1 + t2) + t3;
}

// Whether the entry's alpha >= 1/255 region (Q(d) <= tau, d = pixel centre -
// mean, conic (A, B, C)) meets the rectangle [x0, x1] x [y0, y1] of pixel
// centres. The smallest Q over the rectangle lies on a side facing the mean
// (or is 0 with the mean inside); the comparison is widened by 1e-5 of the
// terms' magnitude so that rounding can only keep a sub-block, never drop one.
__device__ __forceinline__ bool conic_meets_rect(float u, float v, float A, float B, float C, float tau, float x0,
                                                 float x1, float y0, float y1)
{
    const float X0 = x0 - u, X1 = x1 - u, Y0 = y0 - v, Y1 = y1 - v;
    if (X0 <= 0.f && X1 >= 0.f && Y0 <= 0.f && Y1 >= 0.f) return true;
    float q = INFINITY, mag = 0.f, m;
    if (X0 > 0.f || X1 < 0.f) {
        q = conic_edge_min(X0 > 0.f ? X0 : X1, Y0, Y1, A, B, C, __builtin_amdgcn_rcpf(C), m);
        mag = m;
    }
    if (Y0 > 0.f || Y1 < 0.f) {
        const float qy = conic_edge_min(Y0 > 0.f ? Y0 : Y1, X0, X1, C, B, A, __builtin_amdgcn_rcpf(A), m);
        if (qy < q) {
            q = qy;
            mag = m;
        }
    }
    return q <= tau + 1e-5f * mag;
}

// The 16-bit mask of a list entry in its tile (tile origin (tx0, ty0)
// pixels): bit 4 sy + sx is set when the entry's alpha >= 1/255 region may
// touch a pixel centre of the 4x4 sub-block (sx, sy). First the record's
// axis-aligned alpha extent box against the sub-blocks' rectangles of pixel
// centres (clipped to the image; sub-blocks outside it get 0), then the
// ellipse itself against each remaining rectangle, so that an entry is
// dropped from a sub-block only where its alpha is below 1/255 at every
// pixel: skipping it there leaves every result unchanged.
__device__ __forceinline__ uint32_t tile_mask16(const Entry& E, int tx0, int ty0, int W, int H)
{
    const float lo_x = E.a.x - E.c.y, hi_x = E.a.x + E.c.y, lo_y = E.a.y - E.c.z, hi_y = E.a.y + E.c.z;
    float x0[4], x1[4], y0[4], y1[4];
    uint32_t xm = 0, ym = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int bx = tx0 + 4 * k, by = ty0 + 4 * k;
        x0[k] = (float)bx + 0.5f;
        x1[k] = (float)min(bx + 4, W) - 0.5f;
        y0[k] = (float)by + 0.5f;
        y1[k] = (float)min(by + 4, H) - 0.5f;
        xm |= (uint32_t)(bx < W && hi_x >= x0[k] && lo_x <= x1[k]) << k;
        ym |= (uint32_t)(by < H && hi_y >= y0[k] && lo_y <= y1[k]) << k;
    }
    uint32_t mask = 0;
#pragma unroll
    for (int sy = 0; sy < 4; ++sy)
        if ((ym >> sy) & 1u) mask |= xm << (4 * sy);
    if (mask) {
        // the threshold of the record's extent, widened a little more
        const float tau = 2.f * __logf(255.f * E.b.y) * 1.004f + 0.02f;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            if (((mask >> b) & 1u) &&
                !conic_meets_rect(E.a.x, E.a.y, E.a.z, E.a.w, E.b.x, tau, x0[b & 3], x1[b & 3], y0[b >> 2], y1[b >> 2]))
                mask &= ~(1u << b);
        }
    }
    return mask;
}

// As stage_entry, with the record in two vectors (u v -A/2 -B) (-C/2 o r g)
// and blue in its own array.
__device__ __forceinline__ void stage_entry_pair(const Entry& E, int s, float4* __restrict__ s_rec,
                                                 float* __restrict__ s_b, uint8_t* __restrict__ s_mask)
{
    s_rec[2 * s + 0] = make_float4(E.a.x, E.a.y, -0.5f * E.a.z, -E.a.w);
    s_rec[2 * s + 1] = make_float4(-0.5f * E.b.x, E.b.y, E.b.z, E.b.w);
    s_b[s] = E.c.x;
    s_mask[s] = (uint8_t)(E.valid ? E.m4 : 0u);
}

// Per-row compaction of the 64 staged entries: for row r, the slots
// (ascending) whose bit r is set and for which `extra(slot, r)` holds.
// lists[r * 64 + k]; counts in cnt[4] (wave-uniform).
template <typename Pred>
__device__ __forceinline__ void rows_compact(const uint8_t* __restrict__ s_mask, uint16_t* __restrict__ lists,
                                             int lane, uint32_t cnt[4], Pred extra)
{
    asm volatile("" ::: "memory");  // staging writes precede these reads (LDS is in order per wave)
    const uint32_t m4 = s_mask[lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool keep = ((m4 >> r) & 1u) && extra(lane, r);
        const uint64_t m = ballot(keep);
        if (keep) lists[r * RW_BATCH + mask_rank(m)] = (uint16_t)lane;
        cnt[r] = (uint32_t)__popcll(m);
    }
    asm volatile("" ::: "memory");  // list writes precede their reads
}

__device__ __forceinline__ float entry_power(const float4& q0, const float4& q1, float px, float py, float& dx,
                                             float& dy)
{
#pragma clang fp contract(off)
    dx = q0.x - px;
    dy = q0.y - py;
    return __builtin_fmaf(dx, __builtin_fmaf(q0.z, dx, q0.w * dy), (q1.x * dy) * dy);
}

__device__ __forceinline__ int row_max16(int x)
{
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x = max(x, __shfl_xor(x, off));
    return x;
}

struct RasterArgs {
    DevCameras dc;
    int64_t n_blocks;
};

static inline bool raster_args(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                               const uint16_t* masks, const gs_camera* cams, int32_t n_views, const float* bg,
                               RasterArgs& a)
{
    if (n < 0 || !ranges || !bg) return false;
    if (n > 0 && (!rec || !vals || !masks)) return false;
    if (!make_dev_cameras(cams, n_views, a.dc)) return false;
    a.n_blocks = (int64_t)n_views * a.dc.tiles_per_view * 4;
    return a.n_blocks < ((int64_t)1 << 31);
}

}  // namespace gs
