/*
 * gs.h -- C ABI of the MI355X (gfx950) library for one training step of the
 * tile-based differentiable Gaussian rasterizer.
 *
 * The step, in call order:
 *   gs_preprocess          project Gaussians (EWA 2D covariance, SH colour),
 *                          tile rectangles, prefix sum of tile counts
 *   gs_emit_intersections  one (tile, depth) key per Gaussian-tile overlap
 *   gs_sort_keys           LSD radix sort of the keys with their payloads
 *   gs_tile_ranges         [start, end) of each tile in the sorted list
 *   (gs_tile_lists         the three calls above, binned per tile)
 *   gs_tile_masks          per list entry, the 4x4-pixel sub-blocks it touches
 *   gs_rasterize_fwd       front-to-back alpha blending per 16x16 tile
 *   gs_loss_l1             L1 loss against target images, dL/dimage
 *   (gs_rasterize_fwd_l1   the two calls above in one pass)
 *   gs_rasterize_bwd       back-to-front gradients to the 2D quantities
 *   (gs_rasterize_fwd_bwd_l1  gs_rasterize_fwd_l1 and gs_rasterize_bwd in one
 *                          pass)
 *   gs_preprocess_bwd      gradients to all per-Gaussian parameters
 *   gs_adam_step           fused Adam update
 *   (gs_preprocess_bwd_adam  the two calls above in one pass)
 *
 * What the pages fix, and where (the formulas themselves are readings of the
 * 3DGS method, reference [10] of "A Scalable PyTorch Abstraction for Multi-GPU
 * Gaussian Splatting"):
 *   - per-tile sorted lists of Gaussian-to-pixel intersections: "AMD ROCm team
 *     open-sources distributed 3D Gaussian Splatting training for multi-GPU
 *     scaling", section "Distributed training architecture and memory scaling";
 *   - 16x16 pixel blocks: "On Scaling Up 3D Gaussian Splatting Training",
 *     answer (1) on pixel block size;
 *   - 59 fp32 parameters (3 xyz, 3 scale, 4 rotation, 1 opacity, 48 SH): same
 *     page, answer on the storage requirement;
 *   - Adam with two moment vectors (708 bytes per Gaussian): the ROCm page,
 *     same section; Adam is reference [12] of the fVDB page;
 *   - forward and backward rasterization as separate passes whose off-chip
 *     traffic dominates: "ByteSplat: Efficient Distributed 3D Gaussian
 *     Splatting Training via Intra- and Inter-GPU communication reduction",
 *     abstract;
 *   - gradients averaged over a batch of views: "On Scaling Up 3D Gaussian
 *     Splatting Training", answer on the Independent Gradients Hypothesis.
 *
 * Conventions for every entry point
 *   Memory: every array argument is device memory owned by the caller (e.g. a
 *     framework tensor's data pointer), unless marked "host". The library
 *     allocates nothing and keeps no state between calls.
 *   Streams: `stream` is a hipStream_t (NULL = the null stream). Each call
 *     validates its arguments on the host and enqueues kernels on `stream`; it
 *     never synchronises.
 *   Errors: argument errors return GS_ERR_INVALID_ARGUMENT before any HIP call
 *     (so they are testable without a GPU); a failed launch returns GS_ERR_HIP.
 *     Device-side capacity overflow is reported through a device flag.
 *   Parameter block: `params` is [P][n] fp32, structure of arrays, P = 11 +
 *     3 (d+1)^2 for SH degree d (59 at d = 3):
 *       rows 0-2 mean x y z, rows 3-5 log-scale, rows 6-9 quaternion w x y z,
 *       row 10 opacity logit, row 11 + 3k + c SH coefficient k of channel c.
 *     Gradients and the Adam moments use the same layout.
 *   Views: all views of one call share one image size; at most GS_MAX_VIEWS.
 *   Pixels: pixel (i, j) has its centre at (i + 0.5, j + 0.5); images are
 *     [V][3][H][W] fp32, per-pixel maps [V][H][W].
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_ABI_VERSION 2
#define GS_TILE 16
#define GS_MAX_VIEWS 16
#define GS_REC_FLOATS 12 /* floats per projected record */
#define GS_GRAD2D_ROWS 9 /* 2D gradient rows per (view, Gaussian) */

/* `accumulate` flags of gs_rasterize_fwd_bwd_l1 */
#define GS_ACCUMULATE_LOSS 1   /* add to *loss instead of overwriting it */
#define GS_ACCUMULATE_GRAD2D 2 /* add to grad2d instead of zeroing it first */

typedef enum gs_status {
    GS_OK = 0,
    GS_ERR_INVALID_ARGUMENT = 1,
    GS_ERR_CAPACITY = 2,
    GS_ERR_HIP = 3,
    GS_ERR_UNSUPPORTED = 4
} gs_status;

/* Pinhole camera (host memory). World to camera: p_c = R p + t, R row-major;
 * camera axes x right, y down, z forward. A Gaussian is culled unless
 * near_plane < z_c < far_plane (far_plane may be +infinity). */
typedef struct gs_camera {
    int32_t width, height;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    float near_plane, far_plane;
} gs_camera;

/* Projected record of (view v, Gaussian g), rec[(v * n + g) * 12 + field]:
 *   0 u, 1 v          projected mean (pixels)
 *   2 A, 3 B, 4 C     conic = inverse of the 2D covariance [[a, b], [b, c]]
 *                     (EWA: J R Sigma3 R^T J^T plus 0.3 px^2 on the diagonal)
 *   5 opacity         sigmoid of the logit
 *   6 r, 7 g, 8 b     SH colour + 0.5, clamped at 0
 *   9 ext_x, 10 ext_y half-extent of the region where alpha can reach 1/255
 *                     (slightly enlarged; negative when it cannot anywhere)
 *   11 depth          view-space z
 * Written only for visible (view, Gaussian) pairs. */
enum {
    GS_REC_U = 0, GS_REC_V = 1, GS_REC_A = 2, GS_REC_B = 3, GS_REC_C = 4,
    GS_REC_OPACITY = 5, GS_REC_R = 6, GS_REC_G = 7, GS_REC_BLUE = 8,
    GS_REC_EXT_X = 9, GS_REC_EXT_Y = 10, GS_REC_DEPTH = 11
};

/* 2D gradients of (view v, Gaussian g), one 9-float record each:
 * grad2d[(v * n + g) * 9 + row]. */
enum {
    GS_G2_U = 0, GS_G2_V = 1, GS_G2_A = 2, GS_G2_B = 3, GS_G2_C = 4,
    GS_G2_OPACITY = 5, GS_G2_R = 6, GS_G2_G = 7, GS_G2_BLUE = 8
};

int gs_abi_version(void);
const char* gs_status_string(gs_status status);

/* Rows of the parameter block at SH degree d (0..3), or -1. */
int gs_param_rows(int32_t sh_degree);

/* Tiles per row / column / image for one view. */
int32_t gs_tiles_x(int32_t width);
int32_t gs_tiles_y(int32_t height);

/* Number of low key bits the sort must cover: 32 depth bits plus enough bits
 * for every (view, tile) index. */
int32_t gs_sort_end_bit(int32_t n_views, int64_t tiles_per_view);

/* Workspace of gs_preprocess for n Gaussians and V views (bytes). */
size_t gs_preprocess_workspace_bytes(int64_t n, int32_t n_views);

/* Workspace of gs_sort_keys for n_keys keys (bytes). */
size_t gs_sort_workspace_bytes(uint64_t n_keys);

/*
 * gs_preprocess -- the Gaussian-wise stage ("Gaussian-wise computations" of
 * "On Scaling Up 3D Gaussian Splatting Training"; 3D-to-2D transformation).
 * For every view v and Gaussian g: culling (near/far, det <= 0, empty tile
 * rectangle), EWA 2D covariance and its conic, radius ceil(3 sqrt(lambda_max)),
 * tile rectangle [x0, x1) x [y0, y1), SH colour; then an exclusive prefix sum
 * of the per-(v, g) tile counts (the scan is decoupled look-back in
 * reference [21] of the fVDB page; here a reduce-then-scan), or only their
 * total.
 *   params   [P][n] fp32 (P from sh_degree), read only
 *   cams     host array of n_views cameras, all of one image size
 *   rec      out [n_views][n][12] fp32 (see GS_REC_*)
 *   rect     out [n_views][n][4] uint16 x0 y0 x1 y1 (all 0 when culled)
 *   depth    out [n_views][n] fp32, or NULL: the view-space depth of each
 *            entry that is not culled (GS_REC_DEPTH of its record; culled
 *            entries are not written), a compact copy for gs_tile_lists
 *   grad2d   out [n_views][n][9] fp32, or NULL: the 2D-gradient record of
 *            every entry that is not culled is set to zero (the records the
 *            raster passes add to and gs_preprocess_bwd reads; the records of
 *            culled entries are not written), so that the raster passes can
 *            accumulate without a separate clear
 *   offsets  out [n_views * n + 1] uint32: offsets[i] = sum of the tile counts
 *            of entries before i (low 32 bits); the count of entry i is the
 *            area of its rectangle. Or NULL: no counts or offsets are
 *            written and only the total is formed (per-wave sums of the
 *            counts, then their sum), which is all gs_tile_lists needs;
 *            gs_emit_intersections needs the offsets
 *   total    out device uint64: total intersection count K
 *   ws       device workspace of gs_preprocess_workspace_bytes(n, n_views)
 *            (with NULL offsets, 4 ceil(n / 64) bytes suffice)
 * n may be 0. Errors: n < 0, sh_degree outside 0..3, n_views outside
 * 1..GS_MAX_VIEWS, views of different sizes, null pointers (other than the
 * optional ones), small workspace, n_views * tiles_per_view >= 2^31.
 */
gs_status gs_preprocess(const float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                        int32_t n_views, float* rec, uint16_t* rect, float* depth,
                        float* grad2d, uint32_t* offsets, uint64_t* total, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * gs_emit_intersections -- one key per (view, Gaussian, tile) overlap, the
 * per-tile intersection lists of the ROCm page before sorting:
 *   key = ((v * tiles_per_view + ty * tiles_x + tx) << 32) | bits(depth)
 * (bits = IEEE pattern of the fp32 view-space depth, monotone for depth > 0),
 * payload = g. Entry (v, g) writes its count keys at offsets[v * n + g] in
 * row-major tile order.
 *   rec, rect, offsets  from gs_preprocess
 *   keys, vals          out, capacity entries each
 *   overflow            device int32: 1 when an entry would fall at or past
 *                       `capacity` (such entries are not written), else 0
 * Errors: null pointers, n < 0, bad view count.
 */
gs_status gs_emit_intersections(const float* rec, const uint16_t* rect, const uint32_t* offsets,
                                int64_t n, int32_t n_views, int32_t width, int32_t height,
                                uint64_t* keys, uint32_t* vals, uint64_t capacity,
                                int32_t* overflow, void* stream);

/*
 * gs_sort_keys -- stable LSD radix sort (8-bit digits) of n_keys 64-bit keys
 * with uint32 payloads on bits [0, end_bit), the GPU radix sort of reference
 * [22] of the fVDB page. Keys emitted in Gaussian order come out ordered by
 * (key, Gaussian index): a total order, so the result is unique.
 *   keys/vals           in: unsorted; ping buffer
 *   keys_alt/vals_alt   pong buffer of the same size
 *   end_bit             1..64 (gs_sort_end_bit gives the bits a step needs)
 *   ws                  gs_sort_workspace_bytes(n_keys)
 *   result_in_alt       host out: 1 when the sorted data is in the alt pair
 * Errors: null pointers (when n_keys > 0), end_bit outside 1..64, small
 * workspace, n_keys >= 2^32.
 */
gs_status gs_sort_keys(uint64_t* keys, uint32_t* vals, uint64_t* keys_alt, uint32_t* vals_alt,
                       uint64_t n_keys, int32_t end_bit, void* ws, size_t ws_bytes,
                       int32_t* result_in_alt, void* stream);

/* Workspace of gs_tile_lists (bytes) for n Gaussians and a list capacity; 0 on
 * invalid sizes. */
size_t gs_tile_lists_workspace_bytes(int64_t n, int32_t n_views, int32_t width, int32_t height,
                                     uint64_t capacity);

/*
 * gs_tile_lists -- the per-tile intersection lists in depth order and their
 * ranges in one call: the same vals and ranges as gs_emit_intersections,
 * gs_sort_keys and gs_tile_ranges together (the per-tile depth-sorted lists
 * of the ROCm page, section "Distributed training architecture and memory
 * scaling"), built by counting each tile's intersections (LDS counters per
 * chunk of Gaussians), scanning the counts into ranges, filling every tile's
 * slots and sorting each tile's slots by (depth, Gaussian index) on its own.
 *   rec, rect, n, n_views, width, height   as for gs_emit_intersections
 *   depth      the depth output of gs_preprocess, or NULL (then read from
 *              the records): the same lists either way, with less traffic
 *   gauss, gauss_off  device, or NULL: bin only the Gaussians
 *              gauss[gauss_off[v] .. gauss_off[v + 1]) of view v (the output
 *              of gs_window_gaussians for the same window), so that a window
 *              reads only the Gaussians that meet it; the lists are the same
 *              whenever the set holds every Gaussian that meets the window
 *   set_max    with gauss: the most Gaussians a view's set is expected to
 *              hold (0: n), to size the binning grid for the set rather than
 *              for all n Gaussians (a far smaller count table when few are
 *              visible); a larger set is still binned whole, only more
 *              slowly. Must be 0 without gauss.
 *   row0, rows the window of tile rows [row0, row0 + rows) the lists cover
 *              (0 and gs_tiles_y(height) for the whole image): only
 *              intersections with its tiles are listed, so that an image can
 *              be processed band by band with list buffers sized for a band
 *   vals       device out [capacity]: Gaussian ids, tile by tile, front to back
 *   masks      device out [capacity] uint16, or NULL: each entry's sub-block
 *              mask, exactly as gs_tile_masks computes it (written with the
 *              entry's id by the per-tile sorts)
 *   capacity   slots in vals and masks (>= the total of gs_preprocess; < 2^32)
 *   ranges     device out [n_views * tiles_x * rows][2]: [start, end), (0, 0)
 *              if empty, tiles of the window in row-major order per view
 *   overflow   device int32: cleared, then set to 1 if the intersections
 *              exceed capacity (the lists are then incomplete, and the ranges
 *              are cut at capacity so that their readers stay in bounds)
 *   sticky     device int32 or NULL: set to 1 together with overflow, and
 *              never cleared (a flag that outlives the call, e.g. one that
 *              voids every later update until the caller has checked it)
 *   ws         device workspace of gs_tile_lists_workspace_bytes(...)
 * Errors: as gs_emit_intersections, plus a small workspace, capacity >= 2^32,
 * a window outside the tile rows, gauss without gauss_off, set_max < 0 or
 * set_max > 0 without gauss, or more than 8192 tile columns.
 */
gs_status gs_tile_lists(const float* rec, const uint16_t* rect, const float* depth, const uint32_t* gauss,
                        const uint32_t* gauss_off, int64_t set_max, int64_t n, int32_t n_views,
                        int32_t width, int32_t height, int32_t row0, int32_t rows, uint32_t* vals,
                        uint16_t* masks, uint64_t capacity, uint32_t* ranges, int32_t* overflow,
                        int32_t* sticky, void* ws, size_t ws_bytes, void* stream);

/* Workspace of gs_window_gaussians (bytes); 0 on invalid sizes. */
size_t gs_window_gaussians_workspace_bytes(int64_t n, int32_t n_views);

/*
 * gs_window_gaussians -- per view, the Gaussians whose tile rectangle (from
 * gs_preprocess) meets the window of tile rows [row0, row0 + rows), in index
 * order: the set gs_tile_lists needs to bin for that window, so that an image
 * processed window by window (list buffers sized for one window: the
 * per-tile intersection lists are what runs out of memory first at 4K, "AMD
 * ROCm team open-sources distributed 3D Gaussian Splatting training",
 * section "Distributed training architecture and memory scaling") reads
 * only those Gaussians in each window's binning.
 *   rect      [n_views][n][4] uint16 from gs_preprocess
 *   gauss     device out, room for n_views * n ids: view v's members at
 *             gauss[gauss_off[v] ..], ascending
 *   gauss_off device out [n_views + 1]: segment starts, gauss_off[n_views] =
 *             the total
 *   ws        device workspace of gs_window_gaussians_workspace_bytes(n, V)
 * Errors: null pointers, n < 0 or n > 2^31, bad view count, a window outside
 * the tile rows of `height`, a small workspace.
 */
gs_status gs_window_gaussians(const uint16_t* rect, int64_t n, int32_t n_views, int32_t height, int32_t row0,
                              int32_t rows, uint32_t* gauss, uint32_t* gauss_off, void* ws, size_t ws_bytes,
                              void* stream);

/* Workspace of gs_seen_gaussians (bytes); 0 on n < 0. */
size_t gs_seen_gaussians_workspace_bytes(int64_t n);

/*
 * gs_seen_gaussians -- the Gaussians that some view sees (a non-empty
 * rectangle in some view of gs_preprocess's rect), in index order: the set
 * whose gradients gs_preprocess_bwd_compact writes and gs_adam_step_compact
 * reads (the gradients of the visible Gaussians compacted, the single-GPU half
 * of sending only non-zero gradients: ByteSplat abstract).
 *   rect, n, n_views  as for gs_preprocess_bwd
 *   list   device out [n] uint32: the Gaussians, list[0 .. *count)
 *   count  device out uint32: their number
 *   ws     device workspace of gs_seen_gaussians_workspace_bytes(n)
 * Errors: null pointers, n < 0 or n > 2^31, n_views outside [1, 16], a small
 * workspace.
 */
gs_status gs_seen_gaussians(const uint16_t* rect, int64_t n, int32_t n_views, uint32_t* list, uint32_t* count,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * gs_tile_ranges -- for every (view, tile) id t = key >> 32, the range
 * [start, end) of its keys in the sorted list; (0, 0) when it has none.
 *   keys      sorted keys
 *   ranges    out [n_tiles_total][2] uint32 (every entry written)
 * Errors: null pointers, n_keys >= 2^32.
 */
gs_status gs_tile_ranges(const uint64_t* keys, uint64_t n_keys, int64_t n_tiles_total,
                         uint32_t* ranges, void* stream);

/* Bytes of the workspace of gs_tile_masks for lists of `capacity` slots. */
size_t gs_tile_masks_workspace_bytes(uint64_t capacity);

/*
 * gs_tile_masks -- for every entry of the per-tile lists (ranges and vals as
 * produced by gs_tile_ranges / gs_tile_lists), the 16-bit mask of the tile's
 * 4x4-pixel sub-blocks that the entry's alpha >= 1/255 region can touch: bit
 * 4 sy + sx for sub-block (sx, sy), 0 for sub-blocks outside the image. A
 * cleared bit means alpha < 1/255 at every pixel centre of that sub-block,
 * where the blending rule (alpha compositing of the fVDB page: entries with
 * alpha below 1/255 are skipped) leaves the pixel untouched; the raster calls
 * skip those (entry, sub-block) pairs, so their results do not depend on the
 * masks beyond that. The test is the record's alpha-extent box, then the
 * ellipse itself, widened so that rounding only ever sets a bit.
 *   rec, n    records of gs_preprocess
 *   capacity  slots of vals and masks (every range lies below it), < 2^32
 *   masks     out uint16 per list entry, at the entry's list position (slots
 *             in no range are left as they are)
 *   ws        device workspace of gs_tile_masks_workspace_bytes(capacity)
 * Errors: null pointers, bad view count, views of different sizes, a small
 * workspace.
 */
gs_status gs_tile_masks(const float* rec, int64_t n, const uint32_t* ranges, const uint32_t* vals,
                        uint64_t capacity, const gs_camera* cams, int32_t n_views, uint16_t* masks,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * gs_rasterize_fwd -- per pixel, front to back over its tile's sorted list
 * (alpha compositing of the fVDB page; 16x16 tiles):
 *   power = -(A dx^2 + 2 B dx dy + C dy^2) / 2, dx = u - px, dy = v - py;
 *   skip if power > 0; alpha = min(0.99, o exp(power)); skip if alpha < 1/255;
 *   T' = T (1 - alpha); if T' < 1e-4 stop without blending this entry;
 *   otherwise C += rgb alpha T, T = T'.
 *   image     out [V][3][H][W] = C + T_final * bg
 *   T_final   out [V][H][W]
 *   n_contrib out [V][H][W] int32: 1-based list position of the last blended
 *             entry, 0 if none
 *   masks     the lists' sub-block masks of gs_tile_masks
 *   capacity  slots of vals and masks (< 2^32): every range is cut at it and
 *             an id >= n reads as an entry of opacity 0, so that no lists
 *             buffer, however stale, sends a walk outside vals, masks or rec
 *   row0, rows the window of tile rows the lists and ranges cover (as
 *             gs_tile_lists; 0 and gs_tiles_y(height) for the whole image):
 *             only the window's pixels are written
 *   bg        host float[3]
 * Errors: null pointers, bad view count, views of different sizes, a window
 * outside the tile rows.
 */
gs_status gs_rasterize_fwd(const float* rec, int64_t n, const uint32_t* ranges,
                           const uint32_t* vals, const uint16_t* masks, uint64_t capacity,
                           const gs_camera* cams,
                           int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, float* image, float* T_final, int32_t* n_contrib,
                           void* stream);

/*
 * gs_loss_l1 -- L = scale * sum |image - target| over `count` elements and
 * dL/dimage = scale * sign(image - target) (sign(0) = 0). For views averaged
 * over a batch ("On Scaling Up 3D Gaussian Splatting Training", answer on the
 * Independent Gradients Hypothesis) pass scale = 1 / (3 H W V).
 *   loss      device double: overwritten, or added to when `accumulate` is
 *             non-zero
 * Arrays must be 16-byte aligned.
 * Errors: null pointers, count < 0, misaligned arrays.
 */
gs_status gs_loss_l1(const float* image, const float* target, int64_t count, float scale,
                     float* dL_dimage, double* loss, int32_t accumulate, void* stream);

/* Workspace of gs_rasterize_fwd_l1 (bytes): one double per 8x8 quarter of
 * every tile, then the loss reduction's 256 workgroup sums and its arrival
 * counter (2064 bytes; no clearing needed); 0 on invalid sizes. */
size_t gs_rasterize_fwd_l1_workspace_bytes(int32_t n_views, int32_t width, int32_t height);

/*
 * gs_rasterize_fwd_l1 -- gs_rasterize_fwd and gs_loss_l1 in one pass: the
 * same blending (alpha compositing of the fVDB page; 16x16 tiles), then per
 * pixel dL/dimage = scale * sign(I - target) and the loss (+)= scale *
 * sum |I - target| (views averaged as for gs_loss_l1: "On Scaling Up 3D
 * Gaussian Splatting Training", answer on the Independent Gradients
 * Hypothesis). T_final, n_contrib and dL_dimage equal those of the two calls.
 *   capacity  as gs_rasterize_fwd
 *   target    [V][3][H][W]
 *   image     out [V][3][H][W], or null when not wanted
 *   loss      device double: overwritten, or added to when `accumulate`; the
 *             same bits on every call (the partial sums are added in a fixed
 *             order)
 *   ws        device workspace of gs_rasterize_fwd_l1_workspace_bytes(...)
 * Errors: as gs_rasterize_fwd, plus null target / dL_dimage / loss / ws or a
 * small workspace.
 */
gs_status gs_rasterize_fwd_l1(const float* rec, int64_t n, const uint32_t* ranges,
                              const uint32_t* vals, const uint16_t* masks, uint64_t capacity,
                              const gs_camera* cams,
                              int32_t n_views, int32_t row0, int32_t rows,
                              const float* bg, const float* target, float scale, float* image,
                              float* T_final, int32_t* n_contrib, float* dL_dimage, double* loss,
                              int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * gs_rasterize_bwd -- back to front over each pixel's blended entries
 * (backward rasterization of the ByteSplat abstract), gradients to the 2D
 * quantities of every (view, Gaussian):
 *   grad2d  [V][n][9] fp32 (rows GS_G2_*): du dv dA dB dC dopacity dr dg db;
 *           zeroed first unless `accumulate` is non-zero
 * Inputs as in gs_rasterize_fwd (capacity included) plus its T_final and
 * n_contrib and dL/dimage.
 * Floating-point atomics make the summation order, and so the last bits, vary
 * between runs. Errors: as gs_rasterize_fwd.
 */
gs_status gs_rasterize_bwd(const float* rec, int64_t n, const uint32_t* ranges,
                           const uint32_t* vals, const uint16_t* masks, uint64_t capacity,
                           const gs_camera* cams,
                           int32_t n_views, int32_t row0, int32_t rows,
                           const float* bg, const float* T_final, const int32_t* n_contrib,
                           const float* dL_dimage, float* grad2d, int32_t accumulate,
                           void* stream);

/*
 * gs_rasterize_fwd_bwd_l1 -- gs_rasterize_fwd_l1 followed by gs_rasterize_bwd,
 * in one pass per 8x8 quarter of a tile: forward and backward rasterization of
 * the ByteSplat abstract with the L1 loss between them (views averaged as for
 * gs_loss_l1). The L1 gradient of a pixel is a function of that pixel alone,
 * so each quarter blends its pixels, forms dL/dimage and walks its list back
 * with T_final, n_contrib and dL/dimage kept on chip. Results equal those of
 * the two calls (image, T_final, n_contrib, dL/dimage and loss bit for bit;
 * grad2d up to the order of its floating-point atomic additions).
 *   capacity   as gs_rasterize_fwd
 *   target     [V][3][H][W]
 *   image      out [V][3][H][W], or null (not written)
 *   T_final    out [V][H][W], or null
 *   n_contrib  out [V][H][W], or null
 *   dL_dimage  out [V][3][H][W], or null
 *   loss       device double: overwritten, or added to when `accumulate` has
 *              GS_ACCUMULATE_LOSS; the same bits on every call
 *   grad2d     [V][n][9] fp32 as in gs_rasterize_bwd: zeroed first unless
 *              `accumulate` has GS_ACCUMULATE_GRAD2D
 *   ws         device workspace of gs_rasterize_fwd_bwd_l1_workspace_bytes(...):
 *              the per-quarter loss partials and their reduction's sums and
 *              counter, and the order in which the pass takes the tiles
 *              (longest lists first)
 * Errors: as gs_rasterize_fwd, plus null target / loss / ws / grad2d (n > 0),
 * a small workspace or an `accumulate` with other bits than the two flags.
 */
/* Workspace of gs_rasterize_fwd_bwd_l1 (bytes): one double per 8x8 quarter,
 * the loss reduction's 2064 bytes, one 32-bit tile index per tile of every
 * view, and eight 32-bit class counts per 1024 tiles (the longest-first tile
 * order); 0 on invalid sizes. */
size_t gs_rasterize_fwd_bwd_l1_workspace_bytes(int32_t n_views, int32_t width, int32_t height);

gs_status gs_rasterize_fwd_bwd_l1(const float* rec, int64_t n, const uint32_t* ranges,
                                  const uint32_t* vals, const uint16_t* masks, uint64_t capacity,
                                  const gs_camera* cams, int32_t n_views, int32_t row0,
                                  int32_t rows, const float* bg, const float* target, float scale,
                                  float* image, float* T_final, int32_t* n_contrib,
                                  float* dL_dimage, double* loss, float* grad2d,
                                  int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * gs_rasterize_fwd_bwd_l1_noalloc -- gs_rasterize_fwd_bwd_l1 without a
 * workspace argument and without allocating anything, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses that prepare every buffer in advance). Same
 * arguments and results; the workspace is a fixed array of
 * gs_rasterize_fwd_bwd_l1_noalloc_max_bytes() (8 MiB) on each device, which
 * the library holds until the process ends and whose address it looks up on
 * the first call on a device (the device current on the calling thread, which
 * the stream must belong to).
 *   Limit: V x tiles_x x rows tiles with a workspace of at most that size
 *   (36 bytes per tile: about 232,000 tiles, e.g. sixteen 1920x1080 views or
 *   seven 3840x2160 views); larger windows return GS_ERR_CAPACITY before any
 *   HIP call.
 *   Every call on a device uses that device's one array: calls that overlap
 *   on one device (two streams, two threads) race and must be serialised by
 *   the caller. Nothing in the array needs clearing between calls.
 * Errors: as gs_rasterize_fwd_bwd_l1 (without the workspace checks), plus
 * GS_ERR_CAPACITY, and GS_ERR_HIP when the array's address cannot be found.
 */
size_t gs_rasterize_fwd_bwd_l1_noalloc_max_bytes(void);

gs_status gs_rasterize_fwd_bwd_l1_noalloc(const float* rec, int64_t n, const uint32_t* ranges,
                                          const uint32_t* vals, const uint16_t* masks,
                                          uint64_t capacity, const gs_camera* cams, int32_t n_views,
                                          int32_t row0, int32_t rows, const float* bg,
                                          const float* target, float scale, float* image,
                                          float* T_final, int32_t* n_contrib, float* dL_dimage,
                                          double* loss, float* grad2d, int32_t accumulate,
                                          void* stream);

/*
 * gs_preprocess_bwd -- chain rule from the 2D gradients to all P parameters
 * of every Gaussian, summed over views: conic inverse, EWA covariance
 * (including the depth dependence of the Jacobian), projected mean, 3D
 * covariance from scale and rotation, quaternion normalisation, sigmoid,
 * SH colour (coefficients and view direction). Zero where a Gaussian is culled
 * in every view.
 *   grad_params  out [P][n] fp32, overwritten (see `visible`)
 *   visible      device out uint8 [n], or NULL. When given, the output is
 *                sparse: a Gaussian culled in every view reads nothing but
 *                its rectangles, gets visible[g] = 0 and its rows of
 *                grad_params are not written (its gradient is zero); the
 *                others get visible[g] = 1 and their rows. The single-GPU
 *                half of sending only non-zero gradients (the ByteSplat
 *                abstract): gs_adam_step_visible then reads gradients only
 *                where visible[g] is set. NULL: every row written (zeros for
 *                culled Gaussians).
 * Errors: as gs_preprocess.
 */
gs_status gs_preprocess_bwd(const float* params, int64_t n, int32_t sh_degree,
                            const gs_camera* cams, int32_t n_views, const uint16_t* rect,
                            const float* grad2d, float* grad_params, uint8_t* visible,
                            void* stream);

/*
 * gs_preprocess_bwd_adam -- gs_preprocess_bwd followed by gs_adam_step over
 * the [P][n] parameter block, in one pass: each Gaussian's gradient is applied
 * to its parameters and moments as soon as it is formed (same arithmetic as
 * the two calls), so it never goes through device memory.
 *   params       in/out [P][n] fp32: read for the chain rule, then updated
 *   m, v         in/out [P][n] fp32 Adam moments
 *   lr .. step   as gs_adam_step
 *   skip         device int32 or NULL: when non-zero, nothing is written (as
 *                gs_adam_step_unless)
 *   state        device uint8 [n] or NULL: per Gaussian, 0 asserts that its
 *                rows of m and v are all zero. A Gaussian culled in every view
 *                (zero gradient) with state 0 is then skipped without reading
 *                anything: with g = m = v = 0 the update leaves theta, m and v
 *                unchanged when eps > 0 (with eps = 0 the dense update would
 *                write 0/0). Every Gaussian visible in some view gets state 1.
 *                Start it at 0 together with zero moments, or at 1.
 *   grad_params  out [P][n] fp32 or NULL: the gradient, if wanted
 * Errors: as gs_preprocess_bwd and gs_adam_step (m and v must not be null).
 */
gs_status gs_preprocess_bwd_adam(float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                                 int32_t n_views, const uint16_t* rect, const float* grad2d, float* m,
                                 float* v, double lr, double beta1, double beta2, double eps,
                                 int64_t step, const int32_t* skip, uint8_t* state, float* grad_params,
                                 void* stream);

/*
 * gs_adam_step -- Adam (Kingma & Ba, reference [12] of the fVDB page),
 * element-wise over `count` floats, in place:
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   param -= lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps)
 * step is 1-based; beta, 1 - beta, lr / (1 - b1^step) and 1 / sqrt(1 -
 * b2^step) are formed in fp64 on the host and rounded once to fp32.
 * Arrays must be 16-byte aligned.
 * Errors: null pointers, count < 0, step < 1, beta outside [0, 1), eps < 0,
 * misaligned arrays.
 */
gs_status gs_adam_step(float* params, const float* grad, float* m, float* v, int64_t count,
                       double lr, double beta1, double beta2, double eps, int64_t step, void* stream);

/*
 * gs_adam_step_visible -- gs_adam_step over a [rows][n] block whose gradient
 * exists only for the Gaussians with visible[g] set (the sparse output of
 * gs_preprocess_bwd), with the same update arithmetic: the gradient of a
 * Gaussian without the flag is not read (g = 0: its moments still decay and
 * its parameters still move by them, as in the dense update). With `state`
 * (uint8 [n], as in gs_preprocess_bwd_adam: 0 asserts that the Gaussian's
 * moments are zero), a Gaussian without the flag and with state 0 is skipped
 * without reading anything (its update is the identity when eps > 0), and a
 * Gaussian with the flag gets state 1. `skip` (device int32 or NULL): no
 * update at all while it is non-zero (as gs_adam_step_unless).
 * Errors: null pointers, n < 0 or n > 2^31, rows < 1, step < 1, beta outside
 * [0, 1), eps < 0, state with eps = 0.
 */
gs_status gs_adam_step_visible(float* params, const float* grad, float* m, float* v, int64_t n, int32_t rows,
                               const uint8_t* visible, uint8_t* state, double lr, double beta1, double beta2,
                               double eps, int64_t step, const int32_t* skip, void* stream);

/*
 * gs_preprocess_bwd_compact -- gs_preprocess_bwd for the Gaussians of a list
 * (gs_seen_gaussians' output) only, their gradients compacted: Gaussian
 * list[j] (j < *count) gets exactly the gradient gs_preprocess_bwd computes
 * for it, in column j of grad_compact ([rows][stride], rows of
 * gs_param_rows(sh_degree)). The parameter-gradient step of "A Scalable
 * PyTorch Abstraction for Multi-GPU Gaussian Splatting" (reference [10]) as
 * for gs_preprocess_bwd; the compaction is the ByteSplat abstract's (only the
 * non-zero gradients of a step are kept).
 *   list, count  device: the Gaussians and their number
 *   stride       columns of grad_compact (> 0): entries j >= stride are not
 *                written, and *overflow is set when *count > stride
 *   overflow     device int32: set to 1 as above, otherwise left as it is (a
 *                sticky flag: the caller clears it; the skip flag of
 *                gs_adam_step_compact, e.g. gs_tile_lists' sticky flag, so
 *                that a step whose gradients did not fit changes nothing)
 * Errors: as gs_preprocess_bwd, plus stride < 1, null list, count or
 * overflow.
 */
gs_status gs_preprocess_bwd_compact(const float* params, int64_t n, int32_t sh_degree, const gs_camera* cams,
                                    int32_t n_views, const uint16_t* rect, const float* grad2d,
                                    const uint32_t* list, const uint32_t* count, int64_t stride,
                                    float* grad_compact, int32_t* overflow, void* stream);

/*
 * gs_adam_step_compact -- gs_adam_step over a [rows][n] block from the
 * compact gradient of gs_preprocess_bwd_compact (same update arithmetic, so
 * the same bits as gs_adam_step on the dense gradient): Gaussian list[j]
 * (j < min(*count, stride)) is updated with column j of grad_compact; every
 * Gaussian that no view sees (rect, n_views: the Gaussians not in the list
 * when it is gs_seen_gaussians' output for this rect) with g = 0, its moments
 * decaying as in the dense update. With `state` (as in gs_adam_step_visible)
 * an unseen Gaussian with state 0 is skipped without reading anything, and a
 * listed one gets state 1. `skip`: no update at all while non-zero.
 * Errors: null pointers, n < 0 or n > 2^31, rows outside [1, 262140], stride
 * < 1, n_views outside [1, 16], step < 1, beta outside [0, 1), eps < 0, state
 * with eps = 0.
 */
gs_status gs_adam_step_compact(float* params, const float* grad_compact, int64_t stride, const uint32_t* list,
                               const uint32_t* count, float* m, float* v, int64_t n, int32_t rows,
                               const uint16_t* rect, int32_t n_views, uint8_t* state, double lr, double beta1,
                               double beta2, double eps, int64_t step, const int32_t* skip, void* stream);

/*
 * gs_adam_step_unless -- gs_adam_step, skipped on the device when *skip is
 * non-zero (skip: device int32, e.g. the overflow flag of gs_tile_lists, so
 * that a step whose lists did not fit its buffers leaves the parameters and
 * moments untouched and a caller that does not wait for the intersection
 * count can redo it). Errors: as gs_adam_step, plus a null skip.
 */
gs_status gs_adam_step_unless(float* params, const float* grad, float* m, float* v, int64_t count,
                              double lr, double beta1, double beta2, double eps, int64_t step,
                              const int32_t* skip, void* stream);

/*
 * gs_raster_exp -- the exponential the raster passes apply to a pair's power,
 * element-wise: y[i] = 2^fl(x[i] * fl32(log2 e)) on the hardware exp2. The
 * alpha compositing rules (alpha >= 1/255, the 0.99 clamp, T' < 1e-4) are
 * decisions on o exp(power), so a reference implementation that uses another
 * exp must know how far this one may lie from it; this call lets a test
 * measure that.
 *   x, y  device fp32 arrays of n elements (y may alias x)
 * Errors: null pointers (n > 0), n < 0 or n >= 2^40.
 */
gs_status gs_raster_exp(const float* x, float* y, int64_t n, void* stream);

/*
 * gs_stream_copy -- a plain device-to-device copy of `bytes` bytes (16-byte
 * vectors, a grid that fills the chip): it reads and writes exactly 2 x bytes
 * of device memory, the reference for the achievable HBM bandwidth and for
 * scaling the profiler's traffic counters of the other kernels.
 *   dst, src  device memory, 16-byte aligned, not overlapping
 *   bytes     a multiple of 16
 * Errors: null pointers (bytes > 0), misaligned pointers or size.
 */
gs_status gs_stream_copy(void* dst, const void* src, uint64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
