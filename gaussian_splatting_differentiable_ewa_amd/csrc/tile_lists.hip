// gs_tile_lists: the per-tile lists of Gaussian ids in depth order and their
// ranges -- the same result as gs_emit_intersections + gs_sort_keys +
// gs_tile_ranges (per-tile depth-sorted intersection lists, "AMD ROCm team
// open-sources distributed 3D Gaussian Splatting training", section
// "Distributed training architecture and memory scaling"), built by binning
// instead of one global sort of 64-bit keys, with no global atomics:
//   1. k_bin_count    workgroup (view, chunk of about 8192 Gaussians in runs of
//                     16, band of tile rows):
//                     LDS counters of the band's tiles, one increment per
//                     (Gaussian, tile); written as table[view][chunk][tile];
//   2. k_bin_colscan  per (view, tile): exclusive prefix over the chunks (in
//                     place) and the tile's total;
//   3. prefix sum of the totals: each tile's first slot, i.e. its range
//      (k_tl_ranges writes (0, 0) for empty tiles);
//   4. k_bin_fill     the workgroups of step 1 again: LDS cursors start at
//                     tile start + chunk prefix; each (Gaussian, tile) takes
//                     the next slot (LDS atomic) and writes (depth bits, id);
//   5. one wave per tile of up to 64 entries: bitonic sort of the 64-bit
//                     (depth bits, id) across the lanes; one wave per tile
//                     of up to 512 entries (the workgroups of k_tl_sort past
//                     its long tiles take both kinds, four tiles each); and
//      k_tl_sort      one workgroup per longer tile: stable LSD radix sort by
//                     the 32 depth bits (8-bit digits; digits equal across the
//                     tile are skipped), in LDS for up to 4096 entries and
//                     through a global scratch copy beyond; k_tl_ranges lists
//                     its tiles by length class and it takes the longest
//                     first; then runs of equal depth put in id order
//                     (runs longer than TIE_RUN: the whole 64-bit key sorted).
// (depth, id) is a total order, so the arbitrary slot order of step 4 never
// shows: the lists equal those of the global key sort. The positive fp32
// depths order like their bit patterns.
//
// Steps 1 and 4 may take, per view, a set of Gaussians instead of all n (the
// output of gs_window_gaussians: those meeting a window of tile rows, or
// every Gaussian the view sees). With the set's expected size, the grid of
// chunks is sized for the set and its tile rows split into more bands (see
// bin_grid).
//
// With a mask output, each sort kernel also writes every entry's 16-bit
// sub-block mask (gs_tile_masks' test, tile_mask16 in raster_common.h) as it
// writes the entry's id: the record gathers and the test fill the latency of
// the sorts.
#include <algorithm>

#include "raster_common.h"

namespace gs {

constexpr int TL_THREADS = 256;
constexpr int TL_CAP = 4096;                    // entries a tile sorts in LDS
constexpr int TL_ROUNDS = TL_CAP / TL_THREADS;  // rounds of 64 keys per wave, at most
constexpr int GL_CHUNK = 2048;                  // entries per chunk of the global-memory path
constexpr int GL_ROUNDS = GL_CHUNK / TL_THREADS;
constexpr uint32_t GL_RUN = GL_ROUNDS * 64;  // a chunk's items ranked by one wave (a contiguous run)
constexpr int TL_CLASSES = 4;  // length classes of the tiles k_tl_sort takes, longest first
constexpr int WV_CAP = 512;  // entries one wave sorts alone
constexpr int WV_ROUNDS = WV_CAP / 64;
static_assert(4 * WV_CAP <= TL_CAP, "k_tl_sort's LDS holds four one-wave sorts");

constexpr int BAND_TILES = 8192;  // LDS counters of one band of tile rows
// workgroups of a binning grid sized for a set of seen Gaussians (see bin_grid)
constexpr int64_t SET_GRID_WGS = 8192;

struct BinGrid {
    int32_t tiles_x, tiles_y;  // tiles_y: rows of the window of tile rows the lists cover
    int32_t row0;              // the window's first tile row in the image
    int64_t tiles;      // per view, in the window
    int64_t n;          // Gaussians
    int32_t chunks;     // chunks of Gaussians per view
    int64_t chunk;      // Gaussians per chunk
    int32_t band_rows;  // tile rows per band
    int32_t bands;
    // when given, only the Gaussians list[list_off[v] .. list_off[v + 1]) of
    // view v are binned (gs_window_gaussians' output); otherwise all n
    const uint32_t* list;
    const uint32_t* list_off;
};

// the workgroup's (view, chunk, band) and its Gaussians and tile rows. The
// Gaussians are taken in runs of BIN_RUN consecutive ones, and chunk c holds
// runs c, c + chunks, c + 2 chunks, ...: the 64 lanes of a wave then work on
// four places of the scene, not one, whatever the storage order (in a
// spatial order, 64 consecutive Gaussians meet the same tile, and LDS
// atomics on one counter serialise), while each run's rectangles still load
// as one 128-byte piece (runs of 4, 8, 16, 32 measured: 16 and 32 best).
constexpr int64_t BIN_RUN = 16;

struct BinBlock {
    int64_t v, c, len;  // len: local indices of the chunk (some past m in its last run)
    int64_t m;          // Gaussians of the view's set (n, or its list's length)
    const uint32_t* lv; // the view's list, or null
    uint32_t ty0, ty1;
};

// The position in the view's set of local index l of chunk c (may be >= m in
// the last run).
__device__ __forceinline__ int64_t bin_pos(const BinGrid& G, const BinBlock& B, int64_t l)
{
    return ((l / BIN_RUN) * G.chunks + B.c) * BIN_RUN + (l % BIN_RUN);
}

// The Gaussian at position p < m of the view's set.
__device__ __forceinline__ int64_t bin_id(const BinBlock& B, int64_t p) { return B.lv ? (int64_t)B.lv[p] : p; }

__device__ __forceinline__ BinBlock bin_block(const BinGrid& G)
{
    BinBlock B;
    const int64_t per_view = (int64_t)G.chunks * G.bands;
    B.v = blockIdx.x / per_view;
    const int64_t rem = blockIdx.x - B.v * per_view;
    B.c = rem / G.bands;
    const int64_t band = rem - B.c * G.bands;
    if (G.list) {
        const uint32_t o0 = G.list_off[B.v], o1 = G.list_off[B.v + 1];
        B.lv = G.list + o0;
        B.m = o1 > o0 ? (int64_t)(o1 - o0) : 0;
    } else {
        B.lv = nullptr;
        B.m = G.n;
    }
    const int64_t runs = (B.m + BIN_RUN - 1) / BIN_RUN;
    B.len = B.c < runs ? (runs - B.c + G.chunks - 1) / G.chunks * BIN_RUN : 0;
    B.ty0 = (uint32_t)(band * G.band_rows);
    B.ty1 = min((uint32_t)G.tiles_y, B.ty0 + (uint32_t)G.band_rows);
    return B;
}

// a pair's tile rectangle (as stored, image rows), in the window's rows and
// clipped to its rows [ty0, ty1) and the grid
__device__ __forceinline__ bool band_rect(uint2 rr, const BinGrid& G, uint32_t ty0, uint32_t ty1, uint32_t& x0,
                                          uint32_t& y0, uint32_t& x1, uint32_t& y1)
{
    x0 = rr.x & 0xffffu;
    x1 = min(rr.y & 0xffffu, (uint32_t)G.tiles_x);
    const int32_t ly0 = max((int32_t)(rr.x >> 16) - G.row0, (int32_t)ty0);
    const int32_t ly1 = min((int32_t)(rr.y >> 16) - G.row0, (int32_t)ty1);
    y0 = (uint32_t)max(ly0, 0);
    y1 = (uint32_t)max(ly1, 0);
    return x1 > x0 && ly1 > ly0;
}

// Also clears the overflow flag (which k_bin_fill may set), so that no launch
// of its own is needed.
__global__ __launch_bounds__(256) void k_bin_count(const uint16_t* __restrict__ rect, const BinGrid G,
                                                   uint32_t* __restrict__ table, int32_t* __restrict__ overflow)
{
    __shared__ uint32_t cnt[BAND_TILES];
    if (blockIdx.x == 0 && threadIdx.x == 0) *overflow = 0;
    const BinBlock B = bin_block(G);
    const uint32_t nt = (B.ty1 - B.ty0) * (uint32_t)G.tiles_x;
    for (uint32_t i = threadIdx.x; i < nt; i += 256) cnt[i] = 0u;
    __syncthreads();
    // four Gaussians per thread and round: their rectangles are requested
    // together
    for (int64_t l4 = threadIdx.x; l4 < B.len; l4 += 4 * 256) {
        uint2 rr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t l = l4 + 256 * k, p = bin_pos(G, B, l);
            const bool in = l < B.len && p < B.m;
            rr[k] = in ? *(const uint2*)(rect + 4 * (B.v * G.n + bin_id(B, p))) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t x0, y0, x1, y1;
            if (!band_rect(rr[k], G, B.ty0, B.ty1, x0, y0, x1, y1)) continue;
            for (uint32_t ty = y0; ty < y1; ++ty)
                for (uint32_t tx = x0; tx < x1; ++tx) atomicAdd(&cnt[(ty - B.ty0) * G.tiles_x + tx], 1u);
        }
    }
    __syncthreads();
    uint32_t* row = table + (B.v * G.chunks + B.c) * G.tiles + (int64_t)B.ty0 * G.tiles_x;
    for (uint32_t i = threadIdx.x; i < nt; i += 256) row[i] = cnt[i];
}

// 64 tiles per workgroup, each wave one quarter of the chunks: quarter sums,
// then every wave rewrites its quarter as an exclusive prefix
__global__ __launch_bounds__(256) void k_bin_colscan(uint32_t* __restrict__ table, const BinGrid G, int32_t n_views,
                                                     uint32_t* __restrict__ totals, uint32_t* __restrict__ big)
{
    __shared__ uint32_t part[4][64];
    if (blockIdx.x == 0 && threadIdx.x < TL_CLASSES) big[threadIdx.x] = 0u;  // k_tl_ranges counts the classes
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;
    const bool ok = i < (int64_t)n_views * G.tiles;
    const int64_t v = ok ? i / G.tiles : 0, tile = ok ? i - v * G.tiles : 0;
    uint32_t* col = table + v * G.chunks * G.tiles + tile;
    const int32_t q = (G.chunks + 3) / 4, c0 = min((int32_t)w * q, G.chunks), c1 = min(c0 + q, G.chunks);
    // eight chunks' counts are loaded before any is added or rewritten, so
    // that eight loads are in flight (a store may alias the next load
    // otherwise, which serialises them)
    constexpr int CS_BATCH = 8;
    uint32_t sum = 0u;
    if (ok)
        for (int32_t c = c0; c < c1; c += CS_BATCH) {
            uint32_t x[CS_BATCH];
#pragma unroll
            for (int k = 0; k < CS_BATCH; ++k) x[k] = c + k < c1 ? col[(int64_t)(c + k) * G.tiles] : 0u;
#pragma unroll
            for (int k = 0; k < CS_BATCH; ++k) sum += x[k];
        }
    part[w][lane] = sum;
    __syncthreads();
    uint32_t run = 0u;
    for (uint32_t k = 0; k < w; ++k) run += part[k][lane];
    if (ok) {
        for (int32_t c = c0; c < c1; c += CS_BATCH) {
            uint32_t x[CS_BATCH];
#pragma unroll
            for (int k = 0; k < CS_BATCH; ++k) x[k] = c + k < c1 ? col[(int64_t)(c + k) * G.tiles] : 0u;
#pragma unroll
            for (int k = 0; k < CS_BATCH; ++k)
                if (c + k < c1) {
                    col[(int64_t)(c + k) * G.tiles] = run;
                    run += x[k];
                }
        }
        if (w == 3) totals[i] = run;
    }
}

// Length class of a tile that k_tl_sort sorts (more than WV_CAP entries):
// 0 longer than TL_CAP (sorted through global memory), 1 more than 2048, 2
// more than 1024, 3 the rest.
__device__ __forceinline__ int tl_class(uint32_t len)
{
    return len > (uint32_t)TL_CAP ? 0 : len > 2048u ? 1 : len > 1024u ? 2 : 3;
}

// ranges, cut at the capacity: when the lists overflow, readers of the
// ranges stay inside the filled slots. The tiles k_tl_sort sorts are listed
// by length class: class c's count in big[c] (zeroed by k_bin_colscan), its
// tiles in big[TL_CLASSES + c n_tiles + k], so that k_tl_sort takes the
// longest first.
constexpr int TR_THREADS = 1024;

__global__ __launch_bounds__(TR_THREADS) void k_tl_ranges(const uint32_t* __restrict__ starts, int64_t n_tiles,
                                                          uint64_t capacity, uint32_t* __restrict__ ranges,
                                                          uint32_t* __restrict__ big)
{
    __shared__ uint32_t cnt[TL_CLASSES];  // the block's tiles per class, then its first slot per class
    if (threadIdx.x < TL_CLASSES) cnt[threadIdx.x] = 0u;
    const int64_t t = (int64_t)blockIdx.x * TR_THREADS + threadIdx.x;
    const bool ok = t < n_tiles;
    uint32_t s = 0u, e = 0u;
    if (ok) {
        s = (uint32_t)min((uint64_t)starts[t], capacity);
        e = (uint32_t)min((uint64_t)starts[t + 1], capacity);
        *(uint2*)(ranges + 2 * t) = e > s ? make_uint2(s, e) : make_uint2(0u, 0u);
    }
    // one device atomic per class and block (thousands of long tiles on four
    // counters serialise otherwise): LDS slots per wave, then the block's base
    const int c = ok && e > s && e - s > (uint32_t)WV_CAP ? tl_class(e - s) : TL_CLASSES;
    __syncthreads();
    uint32_t slot = 0u;
#pragma unroll
    for (int k = 0; k < TL_CLASSES; ++k) {
        const uint64_t m = ballot(c == k);
        if (!m) continue;
        const uint32_t lead = (uint32_t)__ffsll((unsigned long long)m) - 1u;
        uint32_t first = 0u;
        if (lane_id() == lead) first = atomicAdd(&cnt[k], (uint32_t)__popcll(m));
        first = __shfl(first, (int)lead);
        if (c == k) slot = first + mask_rank(m);
    }
    __syncthreads();
    if (threadIdx.x < TL_CLASSES && cnt[threadIdx.x]) cnt[threadIdx.x] = atomicAdd(big + threadIdx.x, cnt[threadIdx.x]);
    __syncthreads();
    if (c < TL_CLASSES) big[TL_CLASSES + (int64_t)c * n_tiles + cnt[c] + slot] = (uint32_t)t;
}

__global__ __launch_bounds__(256) void k_bin_fill(const float* __restrict__ rec, const uint16_t* __restrict__ rect,
                                                  const float* __restrict__ depth, const BinGrid G, const uint32_t* __restrict__ table,
                                                  const uint32_t* __restrict__ starts, uint2* __restrict__ pairs,
                                                  uint64_t capacity, int32_t* __restrict__ overflow,
                                                  int32_t* __restrict__ sticky)
{
    __shared__ uint32_t cur[BAND_TILES];
    const BinBlock B = bin_block(G);
    const uint32_t nt = (B.ty1 - B.ty0) * (uint32_t)G.tiles_x;
    const int64_t first = (int64_t)B.ty0 * G.tiles_x;
    const uint32_t* row = table + (B.v * G.chunks + B.c) * G.tiles + first;
    const uint32_t* st = starts + B.v * G.tiles + first;
    for (uint32_t i = threadIdx.x; i < nt; i += 256) cur[i] = st[i] + row[i];
    __syncthreads();
    bool over = false;
    for (int64_t l4 = threadIdx.x; l4 < B.len; l4 += 4 * 256) {
        uint2 rr[4];
        uint32_t zb[4], gid[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t l = l4 + 256 * k, p = bin_pos(G, B, l);
            const bool in = l < B.len && p < B.m;
            const int64_t g = in ? bin_id(B, p) : 0, idx = B.v * G.n + g;
            gid[k] = (uint32_t)g;
            rr[k] = in ? *(const uint2*)(rect + 4 * idx) : make_uint2(0u, 0u);
            // the compact depths when given: one float of each 48-byte
            // record would touch every cache line of the records
            zb[k] = !in ? 0u : depth ? __float_as_uint(depth[idx]) : __float_as_uint(rec[idx * GS_REC_FLOATS + GS_REC_DEPTH]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t x0, y0, x1, y1;
            if (!band_rect(rr[k], G, B.ty0, B.ty1, x0, y0, x1, y1)) continue;
            for (uint32_t ty = y0; ty < y1; ++ty)
                for (uint32_t tx = x0; tx < x1; ++tx) {
                    const uint32_t pos = atomicAdd(&cur[(ty - B.ty0) * G.tiles_x + tx], 1u);
                    if (pos < capacity)
                        pairs[pos] = make_uint2(zb[k], gid[k]);
                    else
                        over = true;
                }
        }
    }
    if (over) {
        *overflow = 1;
        if (sticky) *sticky = 1;
    }
}

// Where a kernel writes the id of a tile's entry, its mask too (when wanted).
struct MaskOut {
    uint16_t* masks;
    const float* rec;
    int64_t n;
    int W, H, TX, T, row0;  // T: tiles per view in the window, row0: its first tile row
};

__device__ __forceinline__ void write_mask(const MaskOut& mo, int64_t tile_lin, uint32_t pos, uint32_t id)
{
    if (!mo.masks) return;
    const int64_t view = tile_lin / mo.T;
    const int tile = (int)(tile_lin - view * mo.T);
    const int wy = tile / mo.TX, tx = tile - wy * mo.TX, ty = wy + mo.row0;
    Entry E;
    E.valid = true;
    E.gid = id;
    gather_record(E, mo.rec + view * mo.n * GS_REC_FLOATS, mo.n);
    mo.masks[pos] = (uint16_t)tile_mask16(E, tx * 16, ty * 16, mo.W, mo.H);
}

// The ids of a sorted tile and, when wanted, their masks: positions first,
// first + stride, ... of the tile, MASK_BATCH at a time so that the id reads
// and then the record gathers of that many entries are in flight together.
constexpr int MASK_BATCH = 4;
template <uint32_t STRIDE, typename IdAt>
__device__ __forceinline__ void write_ids_masks(const MaskOut& mo, int64_t tile_lin, uint32_t start, uint32_t n,
                                                uint32_t first, IdAt id_at, uint32_t* __restrict__ vals)
{
    const int64_t view = tile_lin / mo.T;
    const int tile = (int)(tile_lin - view * mo.T);
    const int wy = tile / mo.TX, tx = tile - wy * mo.TX, ty = wy + mo.row0;
    const float* rv = mo.rec + view * mo.n * GS_REC_FLOATS;
    for (uint32_t i0 = first; i0 < n; i0 += MASK_BATCH * STRIDE) {
        Entry E[MASK_BATCH];
#pragma unroll
        for (int k = 0; k < MASK_BATCH; ++k) {
            const uint32_t i = i0 + (uint32_t)k * STRIDE;
            E[k].valid = i < n;
            E[k].gid = E[k].valid ? id_at(i) : 0u;
        }
#pragma unroll
        for (int k = 0; k < MASK_BATCH; ++k)
            if (E[k].valid) vals[start + i0 + (uint32_t)k * STRIDE] = E[k].gid;
        if (!mo.masks) continue;
#pragma unroll
        for (int k = 0; k < MASK_BATCH; ++k) gather_record(E[k], rv, mo.n);
#pragma unroll
        for (int k = 0; k < MASK_BATCH; ++k)
            if (E[k].valid) mo.masks[start + i0 + (uint32_t)k * STRIDE] = (uint16_t)tile_mask16(E[k], tx * 16, ty * 16, mo.W, mo.H);
    }
}

// A tile of up to 64 entries, one wave: a bitonic sort of the 64-bit values
// (depth bits << 32 | id) across the lanes (absent lanes hold the largest
// value and sort last). Run by the workgroups of k_tl_sort past its long
// tiles, four tiles each.
__device__ __forceinline__ void tl_sort_small_tile(int64_t tile, uint32_t lane, const uint32_t* __restrict__ ranges,
                                                   const uint64_t* __restrict__ total_dev, uint64_t capacity,
                                                   const uint2* __restrict__ pairs, uint32_t* __restrict__ vals,
                                                   const MaskOut& mo)
{
    const uint2 rg = *(const uint2*)(ranges + 2 * tile);
    const uint64_t limit = min(capacity, *total_dev);
    const uint32_t start = rg.x, end = (uint32_t)min((uint64_t)rg.y, limit);
    if (end <= start || end - start > 64u) return;  // wave-uniform
    const uint32_t n = end - start;
    uint64_t key = ~0ull;
    if (lane < n) {
        const uint2 p = pairs[start + lane];
        key = ((uint64_t)p.x << 32) | p.y;
    }
    if (n > 1) {
#pragma unroll
        for (uint32_t k = 2; k <= 64; k <<= 1) {
#pragma unroll
            for (uint32_t j = k >> 1; j > 0; j >>= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)key, (int)j), hi = __shfl_xor((uint32_t)(key >> 32), (int)j);
                const uint64_t other = ((uint64_t)hi << 32) | lo;
                const bool up = (lane & k) == 0u;          // this run sorts ascending
                const bool take_min = ((lane & j) == 0u) == up;
                key = take_min ? (other < key ? other : key) : (other > key ? other : key);
            }
        }
    }
    if (lane < n) {
        vals[start + lane] = (uint32_t)key;
        write_mask(mo, tile, start + lane, (uint32_t)key);
    }
}

// lanes of the wave (among `valid`) whose 8-bit digit equals this lane's
__device__ __forceinline__ uint64_t tl_peers(uint32_t d, uint64_t valid)
{
    uint64_t peers = valid;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// Exclusive prefix over the 256 values held one per thread: a scan within
// each wave (shuffles), then the wave totals. Two barriers.
__device__ __forceinline__ uint32_t tl_exclusive_256(uint32_t v, uint32_t* wsum)
{
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (uint32_t off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0;
    for (uint32_t k = 0; k < w; ++k) before += wsum[k];
    __syncthreads();
    return before + x - v;
}

// OR and AND of a value over the workgroup
__device__ __forceinline__ void tl_or_and(uint32_t v_or, uint32_t v_and, uint32_t* s2, uint32_t& o, uint32_t& a)
{
    if (threadIdx.x == 0) {
        s2[0] = 0u;
        s2[1] = 0xffffffffu;
    }
    __syncthreads();
    atomicOr(&s2[0], v_or);
    atomicAnd(&s2[1], v_and);
    __syncthreads();
    o = s2[0];
    a = s2[1];
    __syncthreads();
}

// The sorts order a tile by the 64-bit key (depth bits << 32 | Gaussian id):
// digit positions 0-3 are the id's bytes, 4-7 the depth's, and an LSD pass
// runs for each position whose digit is not the same across the tile. The
// id bytes are sorted only when a tile holds a run of more than TIE_RUN equal
// depths; shorter runs (the only kind that occurs in ordinary scenes) are put
// in id order by an insertion sort after the depth passes, at most
// TIE_RUN^2 / 2 steps per run.
constexpr uint32_t TIE_RUN = 32;

__device__ __forceinline__ uint32_t tl_digit(uint32_t depth, uint32_t id, int p)
{
    return p < 4 ? (id >> (8 * p)) & 255u : (depth >> (8 * (p - 4))) & 255u;
}

// Positions (bits of a mask) whose byte varies, from the OR and AND of the
// values over the tile: 'base' is 0 for the id, 4 for the depth.
__device__ __forceinline__ uint32_t tl_varying(uint32_t vor, uint32_t vand, int base)
{
    const uint32_t differ = vor ^ vand;
    uint32_t m = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        if ((differ >> (8 * b)) & 255u) m |= 1u << (base + b);
    return m;
}

// Orders each run of equal keys (of at most TIE_RUN items) by Gaussian index
// (insertion sort by swaps). Every run is handled by the thread that owns its
// first element; `first`, `stride`: this thread's items.
template <typename KeyAt, typename Less, typename Swap>
__device__ __forceinline__ void tl_fix_short_ties(uint32_t n, uint32_t first, uint32_t stride, KeyAt key_at, Less less,
                                                  Swap swap)
{
    for (uint32_t i = first; i + 1 < n; i += stride) {
        const uint32_t k = key_at(i);
        if ((i > 0 && key_at(i - 1) == k) || key_at(i + 1) != k) continue;
        uint32_t j = i + 1;
        while (j < n && key_at(j) == k) ++j;
        for (uint32_t a = i + 1; a < j; ++a)
            for (uint32_t b = a; b > i && less(b, b - 1); --b) swap(b, b - 1);
    }
}

// LSD passes of one wave over its items key[r] (depth bits) / idx[r]
// (position of the item in the tile's unsorted pairs), item r * 64 + lane,
// through a private slice of LDS (sk, si: WV_CAP items; cnt: 256 counters);
// `positions` the digit positions to sort. The id of an item is read through
// its position (tp[idx].y) for the id passes.
__device__ __forceinline__ void tl_wave_passes(uint32_t n, uint32_t R, uint32_t lane, uint32_t positions,
                                               uint32_t (&key)[WV_ROUNDS], uint32_t (&idx)[WV_ROUNDS], uint32_t* sk,
                                               uint16_t* si, uint32_t* cnt, const uint2* __restrict__ tp)
{
    uint32_t rank[WV_ROUNDS], dig[WV_ROUNDS];
    for (int p = 0; p < 8; ++p) {
        if (((positions >> p) & 1u) == 0u) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) cnt[lane * 4 + k] = 0u;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < WV_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;
            const uint32_t i = (uint32_t)r * 64u + lane;
            const bool valid = i < n;
            dig[r] = valid ? tl_digit(key[r], p < 4 ? tp[idx[r]].y : 0u, p) : 0u;
            const uint64_t peers = tl_peers(dig[r], ballot(valid));
            const uint32_t below = mask_rank(peers);
            const uint32_t prior = cnt[dig[r]];
            rank[r] = prior + below;
            asm volatile("" ::: "memory");
            if (valid && below == 0u) cnt[dig[r]] = prior + (uint32_t)__popcll(peers);
            asm volatile("" ::: "memory");
        }
        // exclusive prefix over the 256 digit counts: four per lane
        uint32_t c[4], sum = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = cnt[lane * 4 + k];
            sum += c[k];
        }
        uint32_t x = sum;
#pragma unroll
        for (uint32_t off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        uint32_t run = x - sum;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            cnt[lane * 4 + k] = run;
            run += c[k];
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < WV_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;
            const uint32_t i = (uint32_t)r * 64u + lane;
            if (i < n) {
                const uint32_t pos = cnt[dig[r]] + rank[r];
                sk[pos] = key[r];
                si[pos] = (uint16_t)idx[r];
            }
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < WV_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;
            const uint32_t i = (uint32_t)r * 64u + lane;
            if (i < n) {
                key[r] = sk[i];
                idx[r] = si[i];
            }
        }
        asm volatile("" ::: "memory");
    }
}

// A tile of 65..512 entries, one wave alone (no barriers: LDS is in order
// within a wave): LSD passes by depth on the wave's registers and a private
// slice of LDS (sk, si: WV_CAP entries, cnt: 256 counters), then the ties.
// Run by the workgroups of k_tl_sort past its long tiles, four tiles each.
__device__ __forceinline__ void tl_sort_wave_tile(int64_t tile, uint32_t lane, uint32_t* sk, uint16_t* si,
                                                  uint32_t* cnt, const uint32_t* __restrict__ ranges,
                                                  const uint64_t* __restrict__ total_dev, uint64_t capacity,
                                                  const uint2* __restrict__ pairs, uint32_t* __restrict__ vals,
                                                  const MaskOut& mo)
{
    const uint2 rg = *(const uint2*)(ranges + 2 * tile);
    const uint64_t limit = min(capacity, *total_dev);
    const uint32_t start = rg.x, end = (uint32_t)min((uint64_t)rg.y, limit);
    if (end <= start) return;
    const uint32_t n = end - start;
    if (n <= 64u || n > (uint32_t)WV_CAP) return;  // wave-uniform
    const uint32_t R = (n + 63u) / 64u;
    const uint2* tp = pairs + start;
    uint32_t key[WV_ROUNDS], idx[WV_ROUNDS];
    uint32_t kor = 0u, kand = 0xffffffffu;
#pragma unroll
    for (int r = 0; r < WV_ROUNDS; ++r) {
        const uint32_t i = (uint32_t)r * 64u + lane;
        key[r] = 0u;
        idx[r] = i;
        if ((uint32_t)r < R && i < n) {
            key[r] = tp[i].x;
            kor |= key[r];
            kand &= key[r];
            sk[i] = key[r];
            si[i] = (uint16_t)i;
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        kor |= __shfl_xor(kor, off);
        kand &= __shfl_xor(kand, off);
    }
    tl_wave_passes(n, R, lane, tl_varying(kor, kand, 4), key, idx, sk, si, cnt, tp);
    // a run of more than TIE_RUN equal depths: sort again by the whole key
    bool longrun = false;
    for (uint32_t i = lane; i + TIE_RUN < n; i += 64) longrun = longrun || sk[i] == sk[i + TIE_RUN];
    if (ballot(longrun) != 0ull) {
        uint32_t ior = 0u, iand = 0xffffffffu;
        for (uint32_t i = lane; i < n; i += 64) {
            const uint32_t id = tp[i].y;
            ior |= id;
            iand &= id;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            ior |= __shfl_xor(ior, off);
            iand &= __shfl_xor(iand, off);
        }
        tl_wave_passes(n, R, lane, tl_varying(ior, iand, 0) | tl_varying(kor, kand, 4), key, idx, sk, si, cnt, tp);
    } else {
        asm volatile("" ::: "memory");
        tl_fix_short_ties(
            n, lane, 64u, [&](uint32_t i) { return sk[i]; },
            [&](uint32_t i, uint32_t a) { return tp[si[i]].y < tp[si[a]].y; },
            [&](uint32_t i, uint32_t a) { const uint16_t x = si[i]; si[i] = si[a]; si[a] = x; });
    }
    asm volatile("" ::: "memory");
    write_ids_masks<64u>(mo, tile, start, n, lane, [&](uint32_t i) { return tp[si[i]].y; }, vals);
}

// LSD passes of the workgroup over a tile of up to TL_CAP items in LDS: wave
// w holds the contiguous run [w L, (w + 1) L), L = 64 R, of items key[r]
// (depth bits) / idx[r] (position in the unsorted pairs tp).
__device__ __forceinline__ void tl_wg_passes(uint32_t n, uint32_t R, uint32_t positions, uint32_t (&key)[TL_ROUNDS],
                                             uint32_t (&idx)[TL_ROUNDS], uint32_t* s_key, uint16_t* s_idx,
                                             uint32_t (*wcnt)[256], uint32_t* s_misc, const uint2* __restrict__ tp)
{
    const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    const uint32_t wbeg = wave * 64u * R;
    // idx[r] holds the item's position (bits 0-11, < TL_CAP); during a pass
    // its rank among the wave's items of its digit (bits 12-22, < 64 R <=
    // 1024) and the digit (bits 23-30) ride in the same register, which keeps
    // the kernel's registers low enough for more waves per SIMD
    static_assert(TL_CAP <= 4096 && TL_ROUNDS * 64 <= 2048, "position and rank fields");
    for (int p = 0; p < 8; ++p) {
        if (((positions >> p) & 1u) == 0u) continue;  // uniform digit: order unchanged
#pragma unroll
        for (int w = 0; w < 4; ++w) wcnt[w][t] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < TL_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;  // uniform across the workgroup
            const uint32_t i = wbeg + (uint32_t)r * 64u + lane;
            const bool valid = i < n;
            const uint32_t pos12 = idx[r] & 0xfffu;
            const uint32_t d = valid ? tl_digit(key[r], p < 4 ? tp[pos12].y : 0u, p) : 0u;
            const uint64_t peers = tl_peers(d, ballot(valid));
            const uint32_t below = mask_rank(peers);
            const uint32_t prior = wcnt[wave][d];
            idx[r] = pos12 | ((prior + below) << 12) | (d << 23);
            asm volatile("" ::: "memory");  // every lane has read the counter
            if (valid && below == 0u) wcnt[wave][d] = prior + (uint32_t)__popcll(peers);
            asm volatile("" ::: "memory");
        }
        __syncthreads();
        {
            const uint32_t c0 = wcnt[0][t], c1 = wcnt[1][t], c2 = wcnt[2][t], c3 = wcnt[3][t];
            const uint32_t lo = tl_exclusive_256(c0 + c1 + c2 + c3, s_misc);
            wcnt[0][t] = lo;
            wcnt[1][t] = lo + c0;
            wcnt[2][t] = lo + c0 + c1;
            wcnt[3][t] = lo + c0 + c1 + c2;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < TL_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;
            const uint32_t i = wbeg + (uint32_t)r * 64u + lane;
            if (i < n) {
                const uint32_t pos = wcnt[wave][idx[r] >> 23] + ((idx[r] >> 12) & 0x7ffu);
                s_key[pos] = key[r];
                s_idx[pos] = (uint16_t)(idx[r] & 0xfffu);
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < TL_ROUNDS; ++r) {
            if ((uint32_t)r >= R) break;
            const uint32_t i = wbeg + (uint32_t)r * 64u + lane;
            if (i < n) {
                key[r] = s_key[i];
                idx[r] = s_idx[i];
            }
        }
    }
}

// LSD passes over a tile longer than the LDS holds, in global memory, chunk
// by chunk (chunks in order keep each pass stable), ping-ponging between src
// and dst (the tile's slots of the pairs and of a scratch copy). One read of
// the list forms the histograms of every position in `positions` (a position
// with one digit across the list is skipped), and each read of a chunk
// requests all its items before ranking them. Returns the buffer that holds
// the result. LDS: hist [8][256], cw [4][256], running [256] (3328 words),
// s_misc.
__device__ __forceinline__ uint2* tl_global_passes(uint32_t n, uint32_t positions, uint2* src, uint2* dst,
                                                   uint32_t* lds, uint32_t* s_misc)
{
    const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    uint32_t(*hist)[256] = (uint32_t(*)[256])lds;           // [position][digit] totals of the list
    uint32_t(*cw)[256] = (uint32_t(*)[256])(lds + 8 * 256);  // [wave][digit] counts of a chunk
    uint32_t* running = lds + 12 * 256;                      // [256] next free slot of each digit
#pragma unroll
    for (int p = 0; p < 8; ++p) hist[p][t] = 0u;
    if (t == 0) s_misc[4] = 0u;
    __syncthreads();
    for (uint32_t base = 0; base < n; base += (uint32_t)GL_CHUNK) {
        uint2 k[GL_ROUNDS];
#pragma unroll
        for (int r = 0; r < GL_ROUNDS; ++r) {
            const uint32_t i = base + wave * GL_RUN + (uint32_t)r * 64u + lane;
            k[r] = i < n ? src[i] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int r = 0; r < GL_ROUNDS; ++r) {
            const uint32_t i = base + wave * GL_RUN + (uint32_t)r * 64u + lane;
            const uint64_t vm = ballot(i < n);
            if (vm == 0ull) break;  // wave-uniform
            for (int p = 0; p < 8; ++p) {
                if (((positions >> p) & 1u) == 0u) continue;
                const uint32_t d = tl_digit(k[r].x, k[r].y, p);
                const uint64_t peers = tl_peers(d, vm);
                if (i < n && mask_rank(peers) == 0u) atomicAdd(&hist[p][d], (uint32_t)__popcll(peers));
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t c = hist[p][t];
        if (((positions >> p) & 1u) && c != 0u && c != n) atomicOr(&s_misc[4], 1u << p);  // two digits or more
    }
    __syncthreads();
    const uint32_t varies = s_misc[4];
    for (int p = 0; p < 8; ++p) {
        if (((varies >> p) & 1u) == 0u) continue;
        running[t] = tl_exclusive_256(hist[p][t], s_misc);
        __syncthreads();
        for (uint32_t base = 0; base < n; base += (uint32_t)GL_CHUNK) {
            // chunk [base, base + GL_CHUNK): wave w ranks its run of GL_RUN
            uint2 item[GL_ROUNDS];
#pragma unroll
            for (int r = 0; r < GL_ROUNDS; ++r) {
                const uint32_t i = base + wave * GL_RUN + (uint32_t)r * 64u + lane;
                item[r] = i < n ? src[i] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) cw[w][t] = 0u;
            __syncthreads();
            uint32_t rk[GL_ROUNDS];
#pragma unroll
            for (int r = 0; r < GL_ROUNDS; ++r) {
                const uint32_t i = base + wave * GL_RUN + (uint32_t)r * 64u + lane;
                const bool valid = i < n;
                const uint32_t d = tl_digit(item[r].x, item[r].y, p);
                const uint64_t peers = tl_peers(d, ballot(valid));
                const uint32_t below = mask_rank(peers);
                const uint32_t prior = cw[wave][d];
                rk[r] = prior + below;
                asm volatile("" ::: "memory");
                if (valid && below == 0u) cw[wave][d] = prior + (uint32_t)__popcll(peers);
                asm volatile("" ::: "memory");
            }
            __syncthreads();
            {
                const uint32_t c0 = cw[0][t], c1 = cw[1][t], c2 = cw[2][t], c3 = cw[3][t];
                const uint32_t b0 = running[t];
                cw[0][t] = b0;
                cw[1][t] = b0 + c0;
                cw[2][t] = b0 + c0 + c1;
                cw[3][t] = b0 + c0 + c1 + c2;
                running[t] = b0 + c0 + c1 + c2 + c3;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < GL_ROUNDS; ++r) {
                const uint32_t i = base + wave * GL_RUN + (uint32_t)r * 64u + lane;
                if (i < n) {
                    const uint32_t pos = cw[wave][tl_digit(item[r].x, item[r].y, p)] + rk[r];
                    if (pos < n) dst[pos] = item[r];
                }
            }
            __syncthreads();
        }
        uint2* tmp = src;
        src = dst;
        dst = tmp;
    }
    return src;
}

// Launched with n_tiles + ceil(n_tiles / 4) workgroups: workgroup b takes
// the b-th tile of the length-class lists of k_tl_ranges, longest class first
// (the workgroups start in about that order, so the long tiles do not finish
// last); the next ceil(n_tiles / 4) take four tiles each, one per wave, and
// sort those of 65..512 entries (tl_sort_wave_tile), filling the chip while
// the long tiles finish, and those of up to 64 (tl_sort_small_tile); the
// rest return.
__global__ __launch_bounds__(TL_THREADS) void k_tl_sort(const uint32_t* __restrict__ ranges, int64_t n_tiles,
                                                        const uint64_t* __restrict__ total_dev, uint64_t capacity,
                                                        uint2* __restrict__ pairs, uint2* __restrict__ alt,
                                                        uint32_t* __restrict__ vals, const uint32_t* __restrict__ big,
                                                        const MaskOut mo)
{
    __shared__ uint32_t s_key[TL_CAP];
    __shared__ uint16_t s_idx[TL_CAP];  // position of each key in the tile's unsorted pairs
    __shared__ uint32_t wcnt[4][256];
    __shared__ uint32_t s_misc[8];
    int64_t tile = -1;
    {
        uint32_t b = blockIdx.x;
#pragma unroll
        for (int c = 0; c < TL_CLASSES; ++c) {
            const uint32_t cnt = big[c];
            if (tile < 0 && b < cnt) tile = big[TL_CLASSES + (int64_t)c * n_tiles + b];
            if (tile < 0) b -= cnt;
        }
        if (tile < 0) {
            const uint32_t wave = threadIdx.x >> 6;
            const int64_t t = (int64_t)b * 4 + wave;
            if (t < n_tiles) {
                tl_sort_small_tile(t, threadIdx.x & 63u, ranges, total_dev, capacity, pairs, vals, mo);
                tl_sort_wave_tile(t, threadIdx.x & 63u, s_key + wave * WV_CAP, s_idx + wave * WV_CAP, wcnt[wave],
                                  ranges, total_dev, capacity, pairs, vals, mo);
            }
            return;
        }
    }
    const uint2 rg = *(const uint2*)(ranges + 2 * (uint64_t)tile);
    const uint64_t limit = min(capacity, *total_dev);
    const uint32_t start = rg.x, end = (uint32_t)min((uint64_t)rg.y, limit);
    if (end <= start) return;
    const uint32_t n = end - start;
    const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    if (n <= (uint32_t)WV_CAP) return;  // tl_sort_small_tile, tl_sort_wave_tile
    const uint2* tp = pairs + start;
    if (n <= (uint32_t)TL_CAP) {
        // wave w holds the contiguous run [w L, (w + 1) L), L = 64 R
        const uint32_t R = (n + TL_THREADS - 1) / TL_THREADS;
        const uint32_t wbeg = wave * 64u * R;
        uint32_t key[TL_ROUNDS], idx[TL_ROUNDS];
        uint32_t kor = 0u, kand = 0xffffffffu;
#pragma unroll
        for (int r = 0; r < TL_ROUNDS; ++r) {
            const uint32_t i = wbeg + (uint32_t)r * 64u + lane;
            const bool valid = (uint32_t)r < R && i < n;
            const uint2 p = valid ? tp[i] : make_uint2(0u, 0u);
            key[r] = p.x;
            idx[r] = i;
            if (valid) {
                kor |= p.x;
                kand &= p.x;
                s_key[i] = p.x;
                s_idx[i] = (uint16_t)i;
            }
        }
        uint32_t o, a;
        tl_or_and(kor, kand, s_misc, o, a);
        tl_wg_passes(n, R, tl_varying(o, a, 4), key, idx, s_key, s_idx, wcnt, s_misc, tp);
        __syncthreads();
        // a run of more than TIE_RUN equal depths: sort again by the whole key
        bool longrun = false;
        for (uint32_t i = t; i + TIE_RUN < n; i += TL_THREADS) longrun = longrun || s_key[i] == s_key[i + TIE_RUN];
        if (__syncthreads_or(longrun)) {
            uint32_t ior = 0u, iand = 0xffffffffu;
            for (uint32_t i = t; i < n; i += TL_THREADS) {
                const uint32_t id = tp[i].y;
                ior |= id;
                iand &= id;
            }
            uint32_t io, ia;
            tl_or_and(ior, iand, s_misc, io, ia);
            tl_wg_passes(n, R, tl_varying(io, ia, 0) | tl_varying(o, a, 4), key, idx, s_key, s_idx, wcnt, s_misc,
                         tp);
        } else {
            tl_fix_short_ties(
                n, t, (uint32_t)TL_THREADS, [&](uint32_t i) { return s_key[i]; },
                [&](uint32_t i, uint32_t a2) { return tp[s_idx[i]].y < tp[s_idx[a2]].y; },
                [&](uint32_t i, uint32_t a2) { const uint16_t x = s_idx[i]; s_idx[i] = s_idx[a2]; s_idx[a2] = x; });
        }
        __syncthreads();
        write_ids_masks<(uint32_t)TL_THREADS>(mo, tile, start, n, t, [&](uint32_t i) { return tp[s_idx[i]].y; },
                                              vals);
        return;
    }

    // a list longer than the LDS holds: the passes over global memory
    uint2* src = tl_global_passes(n, 0xf0u, pairs + start, alt + start, s_key, s_misc);
    __syncthreads();
    // a run of more than TIE_RUN equal depths: sort again by the whole key;
    // otherwise order each (short) run's items by Gaussian index, the keys
    // around eight items per thread requested together
    bool longrun = false;
    for (uint32_t i = t; i + TIE_RUN < n; i += TL_THREADS) longrun = longrun || src[i].x == src[i + TIE_RUN].x;
    if (__syncthreads_or(longrun)) {
        uint2* other = src == pairs + start ? alt + start : pairs + start;
        src = tl_global_passes(n, 0xffu, src, other, s_key, s_misc);
    } else {
        for (uint32_t base = 0; base < n; base += 8u * TL_THREADS) {
            uint32_t kp[8], kc[8], kn[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t i = base + (uint32_t)u * TL_THREADS + t;
                kc[u] = i < n ? src[i].x : 0u;
                kp[u] = i > 0 && i < n ? src[i - 1].x : 0u;
                kn[u] = i + 1 < n ? src[i + 1].x : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t i = base + (uint32_t)u * TL_THREADS + t;
                if (i + 1 >= n || kn[u] != kc[u] || (i > 0 && kp[u] == kc[u])) continue;
                uint32_t j = i + 1;
                while (j < n && src[j].x == kc[u]) ++j;
                for (uint32_t x = i + 1; x < j; ++x)
                    for (uint32_t y = x; y > i && src[y].y < src[y - 1].y; --y) {
                        const uint32_t g = src[y].y;
                        src[y].y = src[y - 1].y;
                        src[y - 1].y = g;
                    }
            }
        }
    }
    __syncthreads();
    write_ids_masks<(uint32_t)TL_THREADS>(mo, tile, start, n, t, [&](uint32_t i) { return src[i].y; }, vals);
}

// workspace: table [V][chunks][T] | totals [V T + 1] | total (u64) | scan
// workspace | pairs [capacity] | scratch pairs [capacity]
struct TlLayout {
    size_t table, totals, total, scan, big, pairs, alt, bytes;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Chunks per view: about 4M table entries in all, at least 1024 Gaussians
// per chunk; sized for m Gaussians per view (m <= 0 or m > n: all n). A set
// larger than m is still binned whole (chunk c takes runs c, c + chunks, ...
// whatever the set's length), with more Gaussians per chunk.
static BinGrid bin_grid(int64_t n, int32_t n_views, int32_t width, int32_t height, int32_t row0 = 0,
                        int32_t rows = -1, int64_t m = 0)
{
    const int64_t ms = (m > 0 && m < n) ? m : n;
    BinGrid G;
    G.tiles_x = gs_tiles_x(width);
    G.tiles_y = rows < 0 ? gs_tiles_y(height) : rows;
    G.row0 = row0;
    G.tiles = (int64_t)G.tiles_x * G.tiles_y;
    G.n = n;
    // Chunks of at most about 8192 Gaussians (at least as many as fill a
    // table of 4M counters), with the table capped at 32M counters and a
    // chunk of at least 1024 Gaussians. A chunk's Gaussians are contiguous in
    // storage, so that their rectangles load coalesced; in a spatial storage
    // order they then meet few tiles, and a large chunk would pile its LDS
    // atomics onto a few counters.
    const int64_t tv = std::max<int64_t>(1, G.tiles * n_views);
    const int64_t want = std::max<int64_t>((ms + 8191) / 8192, ((int64_t)1 << 22) / tv);
    const int64_t cap = std::max<int64_t>(1, ((int64_t)1 << 25) / tv);
    const int64_t by_size = std::max<int64_t>(1, (ms + 1023) / 1024);
    G.chunks = (int32_t)std::min<int64_t>(std::min<int64_t>(want, cap), by_size);
    G.chunk = std::max<int64_t>(1, (ms + G.chunks - 1) / G.chunks);
    G.band_rows = std::max<int32_t>(1, std::min<int32_t>(G.tiles_y, BAND_TILES / G.tiles_x));
    if (m > 0 && m < n) {
        // A grid sized for a set has few chunks, each with many intersections
        // of the same tiles (a set of seen Gaussians is dense on the image):
        // bands of fewer tile rows spread its LDS atomics over about
        // SET_GRID_WGS workgroups instead of a few hundred (city block of 40M
        // Gaussians, 2.2M seen: lists 1.66 -> 0.84 ms; on the whole 1080p
        // headline, more bands cost time, so the other grids keep theirs).
        const int64_t per_band = (int64_t)n_views * G.chunks;
        const int64_t bands = std::max<int64_t>(1, (SET_GRID_WGS + per_band - 1) / per_band);
        G.band_rows = std::min<int32_t>(G.band_rows, (int32_t)std::max<int64_t>(1, (G.tiles_y + bands - 1) / bands));
    }
    G.bands = (G.tiles_y + G.band_rows - 1) / G.band_rows;
    G.list = nullptr;
    G.list_off = nullptr;
    return G;
}

static TlLayout tl_layout(const BinGrid& G, int32_t n_views, uint64_t capacity)
{
    const uint64_t n_tiles = (uint64_t)G.tiles * n_views;
    TlLayout L;
    L.table = 0;
    // the table of any window of rows fits in the larger of the whole
    // image's and 4M counters (a window has fewer tiles and at most as many
    // chunks per 4M counters, or the whole image's table is at the cap too)
    L.totals = align256(std::max<size_t>((size_t)n_tiles * G.chunks, (size_t)1 << 22) * 4);
    L.total = L.totals + align256((n_tiles + 1) * 4);
    L.scan = L.total + 256;
    L.big = L.scan + align256(scan_workspace_bytes(n_tiles));
    L.pairs = L.big + align256((TL_CLASSES + TL_CLASSES * n_tiles) * 4);
    L.alt = L.pairs + align256(capacity * 8);
    L.bytes = L.alt + align256(capacity * 8);
    return L;
}

static bool tl_sizes_ok(int64_t n, int32_t n_views, int32_t width, int32_t height)
{
    if (n < 0 || n_views < 1 || n_views > GS_MAX_VIEWS || width <= 0 || height <= 0) return false;
    if (gs_tiles_x(width) > BAND_TILES || gs_tiles_y(height) > 65535) return false;
    return (int64_t)gs_tiles_x(width) * gs_tiles_y(height) * n_views < ((int64_t)1 << 31);
}

}  // namespace gs

using namespace gs;

extern "C" {

size_t gs_tile_lists_workspace_bytes(int64_t n, int32_t n_views, int32_t width, int32_t height, uint64_t capacity)
{
    if (!tl_sizes_ok(n, n_views, width, height)) return 0;
    return tl_layout(bin_grid(n, n_views, width, height), n_views, capacity).bytes;
}

gs_status gs_tile_lists(const float* rec, const uint16_t* rect, const float* depth, const uint32_t* gauss,
                        const uint32_t* gauss_off, int64_t set_max, int64_t n, int32_t n_views, int32_t width,
                        int32_t height, int32_t row0, int32_t rows, uint32_t* vals, uint16_t* masks,
                        uint64_t capacity, uint32_t* ranges, int32_t* overflow, int32_t* sticky, void* ws,
                        size_t ws_bytes, void* stream)
{
    if (!tl_sizes_ok(n, n_views, width, height)) return GS_ERR_INVALID_ARGUMENT;
    if (row0 < 0 || rows < 1 || row0 + rows > gs_tiles_y(height)) return GS_ERR_INVALID_ARGUMENT;
    if (!ranges || !overflow || !ws) return GS_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!rec || !rect)) return GS_ERR_INVALID_ARGUMENT;
    if (capacity > 0 && !vals) return GS_ERR_INVALID_ARGUMENT;
    if (capacity >= ((uint64_t)1 << 32)) return GS_ERR_INVALID_ARGUMENT;
    if (gauss && !gauss_off) return GS_ERR_INVALID_ARGUMENT;
    if (set_max < 0 || (set_max > 0 && !gauss)) return GS_ERR_INVALID_ARGUMENT;
    // with a set, the grid may be sized for it: its table is then no larger
    // than the whole image's, which the workspace query covers
    BinGrid G = bin_grid(n, n_views, width, height, row0, rows, gauss ? set_max : 0);
    G.list = gauss;
    G.list_off = gauss ? gauss_off : nullptr;
    const TlLayout L = tl_layout(G, n_views, capacity);
    if (ws_bytes < L.bytes) return GS_ERR_INVALID_ARGUMENT;
    const int64_t n_tiles = G.tiles * n_views;
    char* w = (char*)ws;
    uint32_t* table = (uint32_t*)(w + L.table);
    uint32_t* totals = (uint32_t*)(w + L.totals);
    uint64_t* total = (uint64_t*)(w + L.total);
    uint2* pairs = (uint2*)(w + L.pairs);
    uint2* alt = (uint2*)(w + L.alt);
    uint32_t* big = (uint32_t*)(w + L.big);
    hipStream_t s = (hipStream_t)stream;
    const unsigned bin_blocks = (unsigned)((int64_t)n_views * G.chunks * G.bands);
    if (n > 0) {
        hipLaunchKernelGGL(k_bin_count, dim3(bin_blocks), dim3(256), 0, s, rect, G, table, overflow);
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    } else if (fill_u32((uint32_t*)overflow, 1, 0u, s) != hipSuccess ||
               fill_u32(table, (uint64_t)n_tiles * G.chunks, 0u, s) != hipSuccess) {
        return GS_ERR_HIP;
    }
    hipLaunchKernelGGL(k_bin_colscan, dim3(grid_for((uint64_t)n_tiles, 64)), dim3(256), 0, s, table, G, n_views,
                       totals, big);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    if (scan_u32(totals, totals, (uint64_t)n_tiles, total, w + L.scan, s) != hipSuccess) return GS_ERR_HIP;
    hipLaunchKernelGGL(k_tl_ranges, dim3(grid_for((uint64_t)n_tiles, TR_THREADS)), dim3(TR_THREADS), 0, s, totals,
                       n_tiles, capacity, ranges, big);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    if (n == 0) return GS_OK;
    hipLaunchKernelGGL(k_bin_fill, dim3(bin_blocks), dim3(256), 0, s, rec, rect, depth, G, table, totals, pairs,
                       capacity, overflow, sticky);
    if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
    MaskOut mo;
    mo.masks = masks;
    mo.rec = rec;
    mo.n = n;
    mo.W = width;
    mo.H = height;
    mo.TX = G.tiles_x;
    mo.T = (int)G.tiles;
    mo.row0 = row0;
    hipLaunchKernelGGL(k_tl_sort, dim3((unsigned)(n_tiles + grid_for((uint64_t)n_tiles, 4))), dim3(TL_THREADS), 0, s,
                       ranges, n_tiles, total,
                       capacity, pairs, alt, vals, big, mo);
    return hipGetLastError() == hipSuccess ? GS_OK : GS_ERR_HIP;
}

}  // extern "C"
