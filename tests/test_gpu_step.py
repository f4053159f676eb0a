"""The step driver's deferred intersection count on the GPU: steps build the
lists with the capacity they have, Adam is skipped on the device when the
lists overflowed, and the step is redone with larger buffers. Checked by
forcing an overflow with a tiny capacity."""

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import _lib as L
from gaussian_splatting_differentiable_ewa_amd import scenes as S
from gaussian_splatting_differentiable_ewa_amd.step import TrainStep, render, spatial_order

pytestmark = pytest.mark.gpu


def _visible(buf):
    """[V][n] bool: the (view, Gaussian) pairs whose 2D-gradient records the
    step writes (the preprocess zeroes them, the raster adds to them; the
    records of culled pairs are not written)."""
    r = buf.rect.view(buf.V, buf.n, 4).cpu().numpy().view(np.uint16).astype(np.int32)
    return (r[..., 2] > r[..., 0]) & (r[..., 3] > r[..., 1])


def _grad2d_close(a, b, vis_a, vis_b=None, perm_b=None):
    """Visible 2D-gradient records of two steps, equal up to the order of
    their atomic additions (b's Gaussians optionally permuted to a's)."""
    import torch
    assert np.array_equal(vis_a, vis_a if vis_b is None else vis_b)
    V, n = vis_a.shape
    ga = a.grad2d.view(V, n, 9).double()
    gb = b.grad2d.view(V, n, 9).double()
    if perm_b is not None:
        gb = gb[:, torch.from_numpy(perm_b).to(gb.device)]
    m = torch.from_numpy(vis_a).to(ga.device)
    ga, gb = ga[m], gb[m]
    scale = ga.abs().max()
    assert torch.all((ga - gb).abs() <= 1e-4 * ga.abs() + 1e-7 * scale)


def _shrink(b, cap):
    import torch
    b.capacity = cap
    b.vals = torch.empty(cap, dtype=torch.int32, device=b.device)
    b.tl_ws = torch.empty(L.tile_lists_workspace_bytes(b.n, b.V, b.W, b.H, cap), dtype=torch.uint8, device=b.device)


def test_deferred_count_redoes_overflowing_steps():
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[0]
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg)).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    ts = TrainStep(p.clone(), cfg.sh_degree, cams, target, lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps)
    ts.step()  # first step: K read on the host
    ts.flush()
    b = ts.buf
    assert ts.t == 1 and b.path == "binned" and b.lists_without_count()
    after1 = ts.params.clone()
    m1, v1 = ts.m.clone(), ts.v.clone()

    # one overflowing step: Adam is skipped on the device, then redone
    _shrink(b, 16)
    ts.step()
    torch.cuda.synchronize()
    assert int(ts.sticky.item()) == 1
    assert torch.equal(ts.params, after1) and torch.equal(ts.m, m1) and torch.equal(ts.v, v1)
    ts.flush()
    assert ts.t == 1 and ts.redone == 1 and int(ts.sticky.item()) == 0
    assert b.capacity >= b.K > 16
    ts.step()
    ts.flush()
    assert ts.t == 2 and ts.redone == 1
    assert not torch.equal(ts.params, after1)
    assert np.isfinite(float(b.loss.item()))

    # two calls in a row that overflow: the second may find the first's flag
    # already (and run with the new capacity) or not (and be redone too);
    # either way every call is an applied update or a redone one
    _shrink(b, 16)
    t0, r0 = ts.t, ts.redone
    ts.step()
    ts.step()
    ts.flush()
    assert (ts.t - t0) + (ts.redone - r0) == 2
    assert ts.redone > r0 and int(ts.sticky.item()) == 0 and b.capacity >= b.K > 16


def test_compact_gradient_redoes_a_step_that_does_not_fit():
    """The separate backward into the compact gradient: each step's update is
    the dense Adam of the dense gradient of that step's own 2D gradients, bit
    for bit; a step whose seen Gaussians do not fit the buffer sets the sticky
    flag, changes nothing, and is redone with a buffer planned for them."""
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[0]
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg)).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    ts = TrainStep(p.clone(), cfg.sh_degree, cams, target, lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps,
                   fused_adam=False, fused_raster=False, sparse_grad="compact")
    b = ts.buf

    def check_dense(before):
        """ts's state against the dense update from `before` with the step's
        2D gradients (still in the buffers)"""
        th, m, v = (x.clone() for x in before)
        g = torch.empty_like(th)
        L.gs_preprocess_bwd(th, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, g)
        L.gs_adam_step(th, g, m, v, th.numel(), cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, ts.t)
        torch.cuda.synchronize()
        for a, c in ((th, ts.params), (m, ts.m), (v, ts.v)):
            assert torch.equal(a, c)

    start = [x.clone() for x in (ts.params, ts.m, ts.v)]
    ts.step()
    ts.flush()
    assert ts.compact_grad and ts.grad.shape[1] == ts.grad_stride > 16 and b.lists_without_count()
    check_dense(start)
    after1 = [x.clone() for x in (ts.params, ts.m, ts.v)]
    # a buffer of 16 columns: the step is voided on the device, then redone
    ts.grad_stride = 16
    ts.grad = torch.empty((b.P, 16), dtype=torch.float32, device=dev)
    ts.step()
    torch.cuda.synchronize()
    assert int(ts.sticky.item()) == 1
    for a, c in zip(after1, (ts.params, ts.m, ts.v)):
        assert torch.equal(a, c)
    ts.flush()
    assert ts.t == 1 and ts.redone == 1 and int(ts.sticky.item()) == 0 and ts.grad_stride == 0
    ts.step()
    ts.flush()
    before3 = [x.clone() for x in (ts.params, ts.m, ts.v)]
    ts.step()
    ts.flush()
    assert ts.t == 3 and ts.redone == 1 and ts.grad_stride >= int(ts.seen_count.item())
    check_dense(before3)


ZERO_MODES = {
    "default": dict(),
    "separate": dict(fused_raster=False, fused_adam=False),
    "compact-grad": dict(fused_raster=False, fused_adam=False, sparse_grad="compact"),
    "compact-lists": dict(lists="compact"),
    "bands": dict(band_rows=3),
    "budget": dict(list_budget=20_000_000),
}


@pytest.mark.parametrize("mode", list(ZERO_MODES))
def test_zero_gaussians(mode):
    """A scene with no Gaussians (every call takes n = 0) on the odd-size
    views: each pixel is the background, T_final is 1 and n_contrib 0, the
    loss is the oracle's L1 of that image against the target, and the steps
    run and count as applied."""
    import torch

    from oracle import oracle as O
    dev = torch.device("cuda:0")
    cfg = S.RAGGED
    cams = cfg.cameras()
    p = torch.zeros((L.param_rows(cfg.sh_degree), 0), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(5)
    target = rng.random((len(cams), 3, cams[0].height, cams[0].width)).astype(np.float32)
    bg = (0.25, 0.5, 0.75)
    ts = TrainStep(p, cfg.sh_degree, cams, torch.from_numpy(target).to(dev), bg=bg, write_image=True,
                   **ZERO_MODES[mode])
    for _ in range(2):
        ts.step()
    ts.flush()
    torch.cuda.synchronize()
    b = ts.buf
    assert ts.t == 2 and ts.redone == 0 and b.K == 0
    img = b.image.cpu().numpy()
    expect = np.broadcast_to(np.asarray(bg, np.float32)[None, :, None, None], img.shape)
    assert np.array_equal(img, expect)
    if not ts.windowed:  # the windowed step writes these per window, not kept
        assert (b.T_final.cpu().numpy() == 1.0).all() and (b.n_contrib.cpu().numpy() == 0).all()
    loss_o, _ = O.loss_l1(np.ascontiguousarray(expect), target)
    assert float(b.loss.item()) == pytest.approx(loss_o, rel=1e-6)


@pytest.mark.parametrize("fused_raster", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("band_rows", [8, 13])
def test_bands_equal_whole_image(band_rows, fused_raster):
    """The memory-capped mode (lists built and rasterized one window of tile
    rows at a time, 2D gradients and loss summed over the windows) gives the
    image, T_final and n_contrib of the whole-image step bit for bit, and the
    same loss and 2D gradients up to summation order; its list buffers are
    sized for a window."""
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[1]  # 1280x720: 45 tile rows, the last window ragged
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg)).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    kw = dict(lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps, write_image=True, fused_raster=fused_raster)
    whole = TrainStep(p.clone(), cfg.sh_degree, cams, target, **kw)
    banded = TrainStep(p.clone(), cfg.sh_degree, cams, target, band_rows=band_rows, **kw)
    whole.step()
    banded.step()
    whole.flush()
    banded.flush()
    torch.cuda.synchronize()
    a, b = whole.buf, banded.buf
    assert torch.equal(a.image, b.image)
    assert torch.equal(a.T_final, b.T_final)
    assert torch.equal(a.n_contrib, b.n_contrib)
    assert torch.equal(a.dL, b.dL)
    la, lb = float(a.loss.item()), float(b.loss.item())
    assert abs(la - lb) <= 1e-12 * abs(la)
    _grad2d_close(a, b, _visible(a), _visible(b))
    assert b.capacity < a.capacity
    print({"band_rows": band_rows, "whole_slots": a.capacity, "window_slots": b.capacity})


def test_fused_raster_step_equals_separate():
    """A whole-image step with the fused raster pass and one with the separate
    forward + loss and backward calls: image, T_final, n_contrib, dL/dimage
    bit for bit, the loss to rounding and the 2D gradients up to the order of
    their atomic additions."""
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[1]
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg)).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    kw = dict(lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps, write_image=True)
    fused = TrainStep(p.clone(), cfg.sh_degree, cams, target, fused_raster=True, **kw)
    sep = TrainStep(p.clone(), cfg.sh_degree, cams, target, fused_raster=False, **kw)
    fused.step()
    sep.step()
    fused.flush()
    sep.flush()
    torch.cuda.synchronize()
    a, b = fused.buf, sep.buf
    for k in ("image", "T_final", "n_contrib", "dL"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    la, lb = float(a.loss.item()), float(b.loss.item())
    assert abs(la - lb) <= 1e-12 * abs(la)
    _grad2d_close(a, b, _visible(a), _visible(b))


def test_evaluated_pairs_windows_equal_whole_image():
    """The pair count the benchmark reports (from n_contrib, which the fused
    pass keeps on chip) comes from a step of the same mode: in the
    memory-capped mode every window writes its rows; the count equals the
    whole-image step's."""
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[1]
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg)).to(dev)
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    kw = dict(lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps)
    whole = TrainStep(p.clone(), cfg.sh_degree, cams, target, **kw)
    banded = TrainStep(p.clone(), cfg.sh_degree, cams, target, band_rows=13, **kw)
    # the first step of each: both rasterize the same parameters
    a, b = whole.evaluated_pairs(), banded.evaluated_pairs()
    assert a == b and a > 0
    assert whole.t == 1 and banded.t == 1
    # and a second count (a second step) still reads only written rows
    assert banded.evaluated_pairs() > 0 and banded.t == 2


def _tie_tiles(buf):
    """Tiles (view-major index) whose sorted list holds two entries of equal
    depth bits, and the Gaussians listed in them."""
    V, n = buf.V, buf.n
    rng = buf.ranges.view(-1, 2).cpu().numpy().astype(np.int64)
    vals = buf.sorted_vals.cpu().numpy().astype(np.int64)
    z = buf.rec.view(V, n, L.GS_REC_FLOATS)[..., L.REC_DEPTH].cpu().numpy().view(np.uint32)
    lens = rng[:, 1] - rng[:, 0]
    tile = np.repeat(np.arange(rng.shape[0]), lens)
    pos = np.concatenate([np.arange(a, b) for a, b in rng if b > a])
    g = vals[pos]
    d = z[tile // buf.T, g]
    tie = (d[1:] == d[:-1]) & (tile[1:] == tile[:-1])
    tiles = np.unique(tile[1:][tie])
    gauss = np.unique(g[np.isin(tile, tiles)])
    return tiles, gauss


def test_spatial_order_same_step():
    """A step on the Gaussians stored in Morton order (spatial_order) equals
    the step on the generated order, mapped back: the same K; image, T_final
    and n_contrib equal outside the tiles whose list holds two entries of
    equal depth bits (the lists order those by Gaussian index, which the
    permutation changes); 2D gradients (up to the atomics' summation order)
    and updated parameters equal for the Gaussians listed in no such tile."""
    import torch
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[1]
    cams = cfg.cameras()
    p_np = S.make_params(cfg)
    perm = spatial_order(p_np[:3])
    inv = np.argsort(perm)
    assert np.array_equal(np.sort(perm), np.arange(p_np.shape[1]))
    target = render(torch.from_numpy(S.make_target_params(cfg)).to(dev), cfg.sh_degree, cams).clone()
    kw = dict(lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps, write_image=True)
    a = TrainStep(torch.from_numpy(p_np).to(dev), cfg.sh_degree, cams, target, **kw)
    b = TrainStep(torch.from_numpy(np.ascontiguousarray(p_np[:, perm])).to(dev), cfg.sh_degree, cams, target, **kw)
    for ts in (a, b):
        ts.step()
        ts.flush()
    torch.cuda.synchronize()
    assert a.buf.K == b.buf.K > 0
    tiles, gauss = _tie_tiles(a.buf)
    tiles_b, gauss_b = _tie_tiles(b.buf)
    assert np.array_equal(tiles, tiles_b) and np.array_equal(gauss, np.sort(perm[gauss_b]))
    differ = ((a.buf.image != b.buf.image).any(dim=1) | (a.buf.n_contrib != b.buf.n_contrib)
              | (a.buf.T_final != b.buf.T_final)).cpu().numpy()
    V, H, W = differ.shape
    TX = (W + 15) // 16
    vv, jj, ii = np.nonzero(differ)
    where = vv * a.buf.T + (jj // 16) * TX + ii // 16
    print({"pixels_that_differ": int(differ.sum()), "tie_tiles": int(tiles.size), "tie_gaussians": int(gauss.size)})
    assert np.isin(where, tiles).all()
    n = a.buf.n
    keep = np.ones(n, bool)
    keep[gauss] = False
    keep_t = torch.from_numpy(keep).to(dev)
    vis_a = _visible(a.buf)
    assert np.array_equal(vis_a, _visible(b.buf)[:, inv])
    # the written records: visible pairs of Gaussians in no tie tile
    sel = torch.from_numpy(vis_a & keep[None]).to(dev)
    ga = a.buf.grad2d.view(V, n, 9).double()
    gb = b.buf.grad2d.view(V, n, 9).double()[:, torch.from_numpy(inv).to(dev)]
    ga, gb = ga.masked_fill(~sel[..., None], 0.0), gb.masked_fill(~sel[..., None], 0.0)
    # another order of the atomics: 1e-3 relative, with a floor of 1e-5 of
    # each gradient component's largest magnitude (cancelling sums)
    floor = ga.abs().amax(dim=1, keepdim=True)
    err, lim = (ga - gb).abs(), 1e-3 * ga.abs() + 1e-5 * floor
    bad = ~(err <= lim)
    assert not bool(bad.any()), (f"{int(bad.sum())} of {bad.numel()} 2D gradients differ; worst excess "
                                 f"{float((err - lim).max())}; within 1e-4 relative: "
                                 f"{float((err <= 1e-4 * ga.abs()).double().mean())}")
    pa = a.params[:, keep_t]
    pb = b.params[:, torch.from_numpy(inv).to(dev)][:, keep_t]
    # Adam at t = 1 moves each element by about lr sign(g): within 1e-5
    # (|theta| + lr) except where a gradient is summation noise around zero
    close = (pa - pb).abs() <= 1e-5 * (pa.abs() + cfg.lr)
    assert float(close.double().mean()) >= 0.999
