// Shared pieces of the forward and backward raster kernels: the work unit
// (one wavefront per 8x8 quarter of a 16x16 tile), staging of list entries,
// per-row compaction and the fixed-order per-pair arithmetic. The design is
// described in raster_fwd.h.
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

// T: tiles per view in the window of tile rows the launch covers, row0: the
// window's first tile row. `order`, if given, lists the (view, tile)s in the
// order their quarters are taken (the four quarters of a tile stay
// consecutive); otherwise tile order.
__device__ __forceinline__ QuarterCtx quarter_ctx(int W, int H, int TX, int T, int row0,
                                                  const uint32_t* __restrict__ order = nullptr)
{
    QuarterCtx t;
    const uint32_t lb = xcd_chunked(blockIdx.x, gridDim.x);
    const uint32_t quad = lb & 3u;
    t.tile_lin = order ? order[lb >> 2] : lb >> 2;
    t.view = t.tile_lin / (uint32_t)T;
    const uint32_t tile = t.tile_lin - t.view * (uint32_t)T;
    const uint32_t wy = tile / (uint32_t)TX, tx = tile - wy * (uint32_t)TX, ty = wy + (uint32_t)row0;
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

// One list entry on its way from global memory to LDS: its list index (0-based
// within the tile), Gaussian id and quarter bits; valid when the lane holds an
// entry of the batch. Only valid entries are gathered.
struct Entry {
    float4 a, b, c;  // record: (u v A B) (C o r g) (b ex ey z)
    uint32_t gid;
    uint32_t m4;     // the quarter's 4 bits of the entry's tile mask (0 when invalid)
    int32_t rel;
    bool valid;
};

// The quarter's 4 sub-block bits (row r = sub-block (r & 1, r >> 1)) of a
// 16-bit tile mask (bit 4 sy + sx for sub-block (sx, sy) of the tile).
__device__ __forceinline__ uint32_t quarter_bits(uint32_t m16, const QuarterCtx& t)
{
    const uint32_t m = m16 >> t.mshift;
    return (m & 3u) | ((m >> 2) & 0xcu);
}

// ---- Batches of list entries that meet the quarter
// A wave reads its tile's list in chunks of 64 positions (one per lane) and
// keeps only the positions whose mask meets its quarter (about one in four on
// dense scenes). A batch is the compaction, in list order, of the kept
// positions of the longest run of whole chunks (one to four) whose kept
// count fits the 64 lanes, so staged slots are mostly useful ones. The
// quarter bits of the next four chunks are requested one batch ahead.
// Ascending walks (DESC = false) cover list indices 0, 1, ...; descending
// ones (the backward pass) len - 1 down to 0.
struct ChunkScan {
    uint32_t m;    // quarter bits of this lane's position in chunks 0..3, chunk c at bits 4c..4c+3
    int32_t next;  // list index (0-based, within the tile) of lane 0 of chunk 0
};

// The quarter bits of list index `rel` of the tile's list [base, base + len)
// (0 outside it), restricted, when `rl` is given, to the rows whose last
// contributor is at or behind it (1-based position rel + 1 <= rl[r]).
__device__ __forceinline__ uint32_t index_bits(int32_t rel, int32_t len, uint32_t base,
                                               const uint16_t* __restrict__ masks, const QuarterCtx& t,
                                               const int32_t* rl)
{
    if (rel < 0 || rel >= len) return 0u;
    uint32_t m4 = quarter_bits(masks[base + (uint32_t)rel], t);
    if (rl) {
        const int32_t pos = rel + 1;
        m4 &= (pos <= rl[0] ? 1u : 0u) | (pos <= rl[1] ? 2u : 0u) | (pos <= rl[2] ? 4u : 0u) | (pos <= rl[3] ? 8u : 0u);
    }
    return m4;
}

template <bool DESC>
__device__ __forceinline__ int32_t chunk_index(int32_t next, int c, int lane)
{
    return DESC ? next - 64 * c - lane : next + 64 * c + lane;
}

template <bool DESC>
__device__ __forceinline__ ChunkScan scan_start(int32_t first, int32_t len, uint32_t base,
                                                const uint16_t* __restrict__ masks, const QuarterCtx& t,
                                                const int32_t* rl)
{
    ChunkScan S;
    S.next = first;
    S.m = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        S.m |= index_bits(chunk_index<DESC>(first, c, t.lane), len, base, masks, t, rl) << (4 * c);
    return S;
}

// Whether list positions remain from the scan's first chunk on.
template <bool DESC>
__device__ __forceinline__ bool scan_left(const ChunkScan& S, int32_t len)
{
    return DESC ? S.next >= 0 : S.next < len;
}

// The next batch from the scan into E (lane s holds its s-th entry; lanes
// beyond the batch are invalid), with the Gaussian ids requested; returns the
// batch size (wave-uniform). `cs` is 128 bytes of LDS scratch, free between
// the batches' other uses. The scan advances past the chunks taken and
// requests the quarter bits of those that replace them.
template <bool DESC>
__device__ __forceinline__ uint32_t take_batch(ChunkScan& S, Entry& E, int32_t len, uint32_t base,
                                               const uint32_t* __restrict__ vals,
                                               const uint16_t* __restrict__ masks, const QuarterCtx& t,
                                               const int32_t* rl, uint16_t* __restrict__ cs)
{
    uint64_t b[4];
    uint32_t nc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        b[c] = ballot(((S.m >> (4 * c)) & 15u) != 0u);
        nc[c] = (uint32_t)__popcll(b[c]);
    }
    uint32_t j = 1, tot = nc[0];
    if (tot + nc[1] <= 64u) {
        tot += nc[1];
        j = 2;
        if (tot + nc[2] <= 64u) {
            tot += nc[2];
            j = 3;
            if (tot + nc[3] <= 64u) {
                tot += nc[3];
                j = 4;
            }
        }
    }
    // kept positions to their slots, as (offset in the window << 4) | bits
    uint32_t off = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if ((uint32_t)c < j) {
            const uint32_t mc = (S.m >> (4 * c)) & 15u;
            if (mc) cs[off + mask_rank(b[c])] = (uint16_t)(((uint32_t)(64 * c + t.lane) << 4) | mc);
            off += nc[c];
        }
    }
    asm volatile("" ::: "memory");  // scratch writes precede the reads (LDS is in order per wave)
    const uint32_t e = (uint32_t)t.lane < tot ? (uint32_t)cs[t.lane] : 0u;
    asm volatile("" ::: "memory");
    E.valid = (uint32_t)t.lane < tot;
    E.m4 = e & 15u;
    E.rel = DESC ? S.next - (int32_t)(e >> 4) : S.next + (int32_t)(e >> 4);
    E.gid = E.valid ? vals[base + (uint32_t)E.rel] : 0u;
    // advance past the chunks taken and request the ones that replace them
    S.m = j == 4u ? 0u : S.m >> (4 * j);
    S.next = DESC ? S.next - 64 * (int32_t)j : S.next + 64 * (int32_t)j;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if ((uint32_t)c >= 4u - j)
            S.m |= index_bits(chunk_index<DESC>(S.next, c, t.lane), len, base, masks, t, rl) << (4 * c);
    return tot;
}

// An invalid entry gets a zero record (opacity 0): a kernel may evaluate a
// staged slot that no row holds, and must find finite values there. So does
// an id that names no Gaussian (a list buffer the caller never filled): the
// walks stay inside the records whatever the lists hold.
__device__ __forceinline__ void gather_record(Entry& E, const float* __restrict__ rv, int64_t n)
{
    if (E.valid && (int64_t)E.gid < n) {
        const float4* rp = (const float4*)(rv + (int64_t)E.gid * GS_REC_FLOATS);
        E.a = rp[0];
        E.b = rp[1];
        E.c = rp[2];
    } else {
        E.a = E.b = E.c = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Stage the lane's entry at slot `s`: (u, v, -A/2, -B) (-C/2, o, r, g)
// (b, pos, -, -) with pos its 1-based list position (int bits).
__device__ __forceinline__ void stage_entry(const Entry& E, int s, float4* __restrict__ s_rec)
{
    s_rec[3 * s + 0] = make_float4(E.a.x, E.a.y, -0.5f * E.a.z, -E.a.w);
    s_rec[3 * s + 1] = make_float4(-0.5f * E.b.x, E.b.y, E.b.z, E.b.w);
    s_rec[3 * s + 2] = make_float4(E.c.x, __int_as_float(E.rel + 1), 0.f, 0.f);
}

// The 16-bit mask of a list entry in its tile (tile origin (tx0, ty0)
// pixels): bit 4 sy + sx is set when the entry's alpha >= 1/255 region may
// meet the rectangle of pixel centres of the 4x4 sub-block (sx, sy) (clipped
// to the image; sub-blocks outside it get 0). With the conic (A, B, C),
// alpha >= 1/255 is Q(d) = A dx^2 + 2 B dx dy + C dy^2 <= tau = 2 ln(255 o),
// an ellipse. For fixed dy it covers dx = -(B/A) dy -+ w(dy) with w^2 =
// (tau - dy^2 / S_yy) / A (S the 2D covariance, the conic's inverse; S_yy
// comes from the record's y extent, ey = sqrt(tau' S_yy) + 0.05 with the
// preprocess's tau', so no determinant, which cancels for thin footprints,
// is formed). Per row of sub-blocks (a band y0 <= y <= y1) the right end is
// concave in dy and largest at the ellipse's rightmost point dy_R = -(B/C)
// dx_max, dx_max = sqrt(tau S_xx) (from ex likewise), the left end smallest
// at -dy_R: each is taken at that dy clamped into the band, and a sub-block
// is kept when its x range meets the span. tau is widened, w^2 gets a slack
// of a few 1e-6 tau / A (a square root near zero magnifies rounding) and
// the spans a margin of 0.01 px plus a few 1e-6 of the coordinates, so
// rounding can only keep a sub-block: a cleared bit means alpha < 1/255 at
// every pixel centre of the sub-block. (Hardware square roots and
// reciprocals, 1 ulp, are well inside these margins.)
struct MaskGeom {
    float u, v, bA, rA, kY, tau, dym, dyR, mx, my, slack;
    bool ok;  // false: alpha < 1/255 everywhere (or a degenerate record)
};

__device__ __forceinline__ MaskGeom mask_geom(const Entry& E)
{
    MaskGeom M;
    const float u = E.a.x, v = E.a.y, A = E.a.z, B = E.a.w, C = E.b.x, o = E.b.y, ex = E.c.y, ey = E.c.z;
    M.ok = (255.f * o > 1.f) && (ex > 0.05f) && (ey > 0.05f) && (A > 0.f) && (C > 0.f);
    const float l255o = __logf(fmaxf(255.f * o, 1.f));
    M.tau = 2.f * l255o * 1.004f + 0.02f;                // >= the blend threshold's 2 ln(255 o)
    const float tau_rec = 2.f * l255o * 1.002f + 0.01f;  // the extents' threshold
    const float sy = (ey - 0.05f) * (ey - 0.05f) * __builtin_amdgcn_rcpf(tau_rec);  // ~ S_yy
    const float sx = (ex - 0.05f) * (ex - 0.05f) * __builtin_amdgcn_rcpf(tau_rec);  // ~ S_xx
    M.rA = __builtin_amdgcn_rcpf(A);
    M.kY = __builtin_amdgcn_rcpf(sy);
    const float dxm = __builtin_amdgcn_sqrtf(M.tau * sx);
    M.dym = __builtin_amdgcn_sqrtf(M.tau * sy);
    M.mx = 0.01f + 4e-6f * (fabsf(u) + dxm);
    M.my = 0.01f + 4e-6f * (fabsf(v) + M.dym);
    M.slack = 4e-6f * M.tau * M.rA;
    M.dyR = -B * dxm * __builtin_amdgcn_rcpf(C);
    M.bA = B * M.rA;
    M.u = u;
    M.v = v;
    return M;
}

// The ellipse's x span [xl, xr] inside the band of pixel-centre rows
// [yc0, yc1]; false when the band misses it.
__device__ __forceinline__ bool band_span(const MaskGeom& M, float yc0, float yc1, float& xl, float& xr)
{
    const float a = fmaxf(yc0 - M.v - M.my, -M.dym - M.my);
    const float b = fminf(yc1 - M.v + M.my, M.dym + M.my);
    if (!(a <= b)) return false;
    const float dR = fminf(fmaxf(M.dyR, a), b), dL = fminf(fmaxf(-M.dyR, a), b);
    const float wR = __builtin_amdgcn_sqrtf(fmaxf((M.tau - dR * dR * M.kY) * M.rA, 0.f) + M.slack);
    const float wL = __builtin_amdgcn_sqrtf(fmaxf((M.tau - dL * dL * M.kY) * M.rA, 0.f) + M.slack);
    xr = M.u - M.bA * dR + wR + M.mx;
    xl = M.u - M.bA * dL - wL - M.mx;
    return true;
}

// Bits of the four sub-block columns from pixel tx0 whose pixel-centre
// range [tx0 + 4k + 0.5, min(tx0 + 4k + 4, W) - 0.5] meets [xl, xr]
// (columns outside the image never): k runs from the first column whose
// right centre is >= xl to the last whose left centre is <= xr.
__device__ __forceinline__ uint32_t span_cols(float xl, float xr, int tx0, int W)
{
    if (xl > (float)W - 0.5f) return 0u;  // right of every pixel centre (and of a clipped last column)
    const float base = (float)tx0;
    const int khi = (int)floorf(fminf(fmaxf((xr - base - 0.5f) * 0.25f, -8.f), 8.f));
    const int klo = (int)ceilf(fminf(fmaxf((xl - base - 3.5f) * 0.25f, -8.f), 8.f));
    const int hi = min(khi, min(3, ((W - tx0 + 3) >> 2) - 1)), lo = max(klo, 0);
    return hi < lo ? 0u : ((2u << hi) - 1u) & ~((1u << lo) - 1u);
}

// The pixel-centre rows of sub-block row r of the tile row starting at ty0.
__device__ __forceinline__ bool band_rows(int ty0, int r, int H, float& yc0, float& yc1)
{
    const int by = ty0 + 4 * r;
    yc0 = (float)by + 0.5f;
    yc1 = (float)min(by + 4, H) - 0.5f;
    return by < H;
}

__device__ __forceinline__ uint32_t tile_mask16(const Entry& E, int tx0, int ty0, int W, int H)
{
    const MaskGeom M = mask_geom(E);
    if (!M.ok) return 0u;
    uint32_t mask = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float yc0, yc1, xl, xr;
        if (!band_rows(ty0, r, H, yc0, yc1)) break;
        if (!band_span(M, yc0, yc1, xl, xr)) continue;  // the band misses the ellipse
        mask |= span_cols(xl, xr, tx0, W) << (4 * r);
    }
    return mask;
}

// As stage_entry, with the record in two vectors (u v -A/2 -B) (-C/2 o r g)
// and (blue, pos) in an array of their own.
__device__ __forceinline__ void stage_entry_pair(const Entry& E, int s, float4* __restrict__ s_rec,
                                                 float2* __restrict__ s_bp)
{
    s_rec[2 * s + 0] = make_float4(E.a.x, E.a.y, -0.5f * E.a.z, -E.a.w);
    s_rec[2 * s + 1] = make_float4(-0.5f * E.b.x, E.b.y, E.b.z, E.b.w);
    s_bp[s] = make_float2(E.c.x, __int_as_float(E.rel + 1));
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

// A tile's list [start, end) from the ranges, cut at the list capacity: a
// stale or foreign ranges buffer cannot send a walk outside vals and masks.
__device__ __forceinline__ uint2 tile_range(const uint32_t* __restrict__ ranges, uint32_t tile_lin, uint32_t cap)
{
    uint2 rg = *(const uint2*)(ranges + 2 * (uint64_t)tile_lin);
    rg.y = min(rg.y, cap);
    rg.x = min(rg.x, rg.y);
    return rg;
}

struct RasterArgs {
    DevCameras dc;
    int32_t row0, T;  // the window of tile rows: first row, tiles per view
    int64_t n_blocks;
    uint32_t cap;     // slots of vals and masks
};

static inline bool raster_args(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                               const uint16_t* masks, uint64_t capacity, const gs_camera* cams, int32_t n_views,
                               int32_t row0, int32_t rows, const float* bg, RasterArgs& a)
{
    if (n < 0 || !ranges || !bg) return false;
    if (capacity >= ((uint64_t)1 << 32)) return false;
    if (capacity > 0 && (!vals || !masks)) return false;
    if (n > 0 && !rec) return false;
    if (!make_dev_cameras(cams, n_views, a.dc)) return false;
    if (row0 < 0 || rows < 1 || row0 + rows > a.dc.tiles_y) return false;
    a.row0 = row0;
    a.T = a.dc.tiles_x * rows;
    a.n_blocks = (int64_t)n_views * a.T * 4;
    a.cap = (uint32_t)capacity;
    return a.n_blocks < ((int64_t)1 << 31);
}

}  // namespace gs
