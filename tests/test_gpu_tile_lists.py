"""gs_tile_lists through the C ABI against the oracle's emission and library
sort (ordered by tile, depth bits, Gaussian index) on synthetic rectangles
and depths built to stress it: many equal depths (the order of equal depths
is decided by the index), every depth equal (tiles that are one run of ties,
of hundreds to thousands of entries), tiles with more entries than one
workgroup sorts in LDS (4096: their passes run over global memory in chunks,
several chunks per tile), empty tiles and views, and a capacity with slack."""

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import _lib as L
from oracle import oracle as O

pytestmark = pytest.mark.gpu

W, H = 256, 192  # 16 x 12 tiles


def _scene(seed, n, V, big_share, depth_levels):
    rng = np.random.default_rng(seed)
    TX, TY = (W + 15) // 16, (H + 15) // 16
    rect = np.zeros((V, n, 4), np.int32)
    for v in range(V):
        x0 = rng.integers(0, TX, n)
        y0 = rng.integers(0, TY, n)
        w = rng.integers(0, 4, n)  # width 0 culls the Gaussian in this view
        h = rng.integers(1, 4, n)
        big = rng.random(n) < big_share[v]
        x0[big], y0[big], w[big], h[big] = 0, 0, TX, TY
        rect[v, :, 0], rect[v, :, 1] = x0, y0
        rect[v, :, 2], rect[v, :, 3] = np.minimum(x0 + w, TX), np.minimum(y0 + h, TY)
    vis = ((rect[..., 2] > rect[..., 0]) & (rect[..., 3] > rect[..., 1])).astype(np.uint8)
    if depth_levels:
        z = rng.choice(np.linspace(0.5, 60.0, depth_levels).astype(np.float32), (V, n))
    else:
        z = rng.uniform(0.02, 200.0, (V, n)).astype(np.float32)
    rec = np.zeros((V, n, L.GS_REC_FLOATS), np.float32)
    rec[..., L.REC_DEPTH] = z
    return rect, vis, z.astype(np.float32), rec, TX, TY


CASES = [
    # seed, n, views, share of whole-image rectangles per view, depth levels
    (1, 3000, 1, (0.0,), 0),
    (2, 3000, 2, (0.0, 0.0), 12),        # heavy ties
    (3, 9000, 2, (0.6, 0.0), 0),         # view 0: every tile > 4096 entries
    (4, 9000, 2, (0.55, 0.02), 7),       # long lists with heavy ties
    (5, 500, 3, (0.0, 1.0, 0.0), 3),     # every Gaussian in every tile of view 1
    (6, 20000, 1, (0.45,), 0),           # every tile > 8192 entries: the global-memory path, 5 chunks
    (7, 14000, 2, (0.0, 0.5), 9),        # view 1: 7000-entry tiles over global memory, with ties
    # every Gaussian at one depth (a wall facing the camera): each tile's list
    # is one run of equal depths, ordered by index alone -- with one wave
    # (about 300 entries per tile), one workgroup in LDS (about 2700) and the
    # global-memory path (about 8100)
    (8, 1500, 1, (0.2,), 1),
    (9, 3000, 1, (0.9,), 1),
    (10, 9000, 1, (0.9,), 1),
]


@pytest.mark.parametrize("seed,n,V,big,levels", CASES)
def test_tile_lists_match_oracle(seed, n, V, big, levels):
    import torch
    dev = torch.device("cuda:0")
    rect, vis, z, rec, TX, TY = _scene(seed, n, V, big, levels)
    rect[vis == 0] = 0  # culled pairs carry an empty rectangle, as preprocess writes them
    keys, vals = O.emit_sorted(rect, vis, z, TX, TY)
    ranges = O.tile_ranges(keys, V * TX * TY)
    K = vals.size
    print(f"[tile_lists] seed {seed}: K {K}, longest list {int((ranges[:, 1] - ranges[:, 0]).max())}", flush=True)
    rec_t = torch.from_numpy(rec.reshape(-1)).to(dev)
    rect_t = torch.from_numpy(rect.astype(np.int16).reshape(-1)).to(dev)
    # the depths from the records, or from a compact copy (culled pairs hold
    # garbage there, as preprocess leaves them)
    depth = rec.reshape(-1, L.GS_REC_FLOATS)[:, L.REC_DEPTH].copy()
    depth[vis.reshape(-1) == 0] = np.nan
    depth_t = torch.from_numpy(depth).to(dev)
    for cap, dep in ((K, None), (K + 1000, None), (K, depth_t)):
        out = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=dev)
        rng_t = torch.full((V * TX * TY * 2,), -1, dtype=torch.int32, device=dev)
        ovf = torch.full((1,), 5, dtype=torch.int32, device=dev)
        ws = torch.empty(L.tile_lists_workspace_bytes(n, V, W, H, cap), dtype=torch.uint8, device=dev)
        L.gs_tile_lists(rec_t, rect_t, n, V, W, H, out, cap, rng_t, ovf, ws, depth=dep)
        torch.cuda.synchronize()
        assert int(ovf.item()) == 0
        assert np.array_equal(out.cpu().numpy()[:K].view(np.uint32), vals)
        assert np.array_equal(rng_t.cpu().numpy().view(np.uint32).reshape(-1, 2), ranges)


WINDOW_CASES = [
    # seed, n, views, big share, depth levels, windows of tile rows
    (11, 3000, 2, (0.1, 0.0), 0, [(0, 5), (5, 5), (10, 2)]),
    (12, 9000, 1, (0.3,), 5, [(0, 1), (1, 7), (8, 4)]),
    (13, 2000, 3, (0.0, 0.5, 0.0), 0, [(3, 4), (11, 1)]),
]


@pytest.mark.parametrize("seed,n,V,big,levels,windows", WINDOW_CASES)
def test_window_sets_and_lists(seed, n, V, big, levels, windows):
    """gs_window_gaussians lists, per view and in index order, exactly the
    Gaussians whose rectangle meets the window's tile rows; gs_tile_lists fed
    that set gives, bit for bit, the oracle's lists of the window's tiles
    (the whole-image key list restricted to those rows), and the same lists
    as without the set."""
    import torch
    dev = torch.device("cuda:0")
    rect, vis, z, rec, TX, TY = _scene(seed, n, V, big, levels)
    rect[vis == 0] = 0
    keys, vals = O.emit_sorted(rect, vis, z, TX, TY)
    tile = (keys >> np.uint64(32)).astype(np.int64)
    view, t = tile // (TX * TY), tile % (TX * TY)
    ty, tx = t // TX, t % TX
    rec_t = torch.from_numpy(rec.reshape(-1)).to(dev)
    rect_t = torch.from_numpy(rect.astype(np.int16).reshape(-1)).to(dev)
    gauss = torch.full((V * n,), -1, dtype=torch.int32, device=dev)
    off = torch.full((V + 1,), -1, dtype=torch.int32, device=dev)
    wws = torch.empty(L.window_gaussians_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    for row0, rows in windows:
        # the window's Gaussian sets against a host compaction
        L.gs_window_gaussians(rect_t, n, V, H, row0, rows, gauss, off, wws)
        torch.cuda.synchronize()
        o = off.cpu().numpy().astype(np.int64)
        g = gauss.cpu().numpy()
        meets = (vis == 1) & (rect[..., 1] < row0 + rows) & (rect[..., 3] > row0)
        assert o[0] == 0 and o[V] == int(meets.sum())
        for v in range(V):
            assert np.array_equal(g[o[v]:o[v + 1]], np.nonzero(meets[v])[0])
        # the oracle's lists of the window's tiles, in window-local tile order
        sel = (ty >= row0) & (ty < row0 + rows)
        wtile = view[sel] * (TX * rows) + (ty[sel] - row0) * TX + tx[sel]
        wkeys = (wtile.astype(np.uint64) << np.uint64(32)) | (keys[sel] & np.uint64(0xffffffff))
        wvals = vals[sel]
        wranges = O.tile_ranges(wkeys, V * TX * rows)
        K = wvals.size
        for with_set in (True, False):
            cap = K + 64
            out = torch.full((cap,), -1, dtype=torch.int32, device=dev)
            rng_t = torch.full((V * TX * rows * 2,), -1, dtype=torch.int32, device=dev)
            ovf = torch.full((1,), 5, dtype=torch.int32, device=dev)
            ws = torch.empty(L.tile_lists_workspace_bytes(n, V, W, 16 * rows, cap), dtype=torch.uint8, device=dev)
            L.gs_tile_lists(rec_t, rect_t, n, V, W, H, out, cap, rng_t, ovf, ws, row0=row0, rows=rows,
                            gauss=gauss if with_set else None, gauss_off=off if with_set else None)
            torch.cuda.synchronize()
            assert int(ovf.item()) == 0
            assert np.array_equal(out.cpu().numpy()[:K].view(np.uint32), wvals), (row0, rows, with_set)
            assert np.array_equal(rng_t.cpu().numpy().view(np.uint32).reshape(-1, 2), wranges), (row0, rows, with_set)
        print(f"[tile_lists] seed {seed} window {row0}+{rows}: {K} entries, set {o[V]} of {V * n}", flush=True)
