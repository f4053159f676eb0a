"""Parity harness: runs the HIP path stage by stage through the C ABI and the
CPU oracle on the same seeded inputs, and compares them (used by the GPU tests,
the smoke check and the benchmark's sampled check).

Tolerances (fp32 throughout; the oracle accumulates gradients in fp64):
  * integer stages -- counts, offsets, K, keys, order, ranges, n_contrib at
    unambiguous pixels: bit-exact;
  * image: max abs 1e-4 at pixels the oracle does not flag as ambiguous (an
    alpha within the exp() rounding band of 1/255, or a T' within the
    propagated band of 1e-4: there a last-ulp exp() difference may flip a
    discrete decision, and both answers are correct);
  * 2D gradients (both sides fed the same dL/dimage, zero at ambiguous
    pixels): |g - g_ref| <= 1e-3 |g_ref| + 1e-4 A_ref, A_ref the sum of the
    absolute contributions (fp32 atomics reorder cancelling sums);
  * parameter gradients, fed the same 2D gradients: 1e-3 relative with a floor
    of 1e-6 x the row's largest magnitude (fp32 cancellation in the chain rule);
  * Adam, fed the same gradients: 1e-5 relative, floors 1e-5 (|ref| + lr) for
    parameters and 1e-5 (|b1 m| + |(1 - b1) g|) for the first moment.
"""

from __future__ import annotations

import numpy as np
import torch

from gaussian_splatting_differentiable_ewa_amd import _lib as L
from gaussian_splatting_differentiable_ewa_amd.step import Buffers
from oracle import oracle as O

IMAGE_ATOL = 1e-4
GRAD_RTOL, GRAD_AFLOOR = 1e-3, 1e-4
PGRAD_RTOL, PGRAD_ROWFLOOR = 1e-3, 1e-6
ADAM_RTOL = 1e-5


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_forward(params_np: np.ndarray, sh: int, cams, bg=(0.0, 0.0, 0.0)):
    """Preprocess, keys, sort, ranges and forward raster on the GPU. Returns
    the Buffers object (device state kept for the backward) and host copies."""
    dev = torch.device("cuda:0")
    p = torch.from_numpy(np.ascontiguousarray(params_np)).to(dev)
    b = Buffers(p.shape[1], sh, cams, device=dev, lists="binned", offsets=True)
    b.preprocess(p)
    torch.cuda.synchronize()
    out = {"params_t": p,
           "rec": np_(b.rec).reshape(b.V, b.n, L.GS_REC_FLOATS),
           "rect": np_(b.rect).view(np.uint16).reshape(b.V, b.n, 4).astype(np.int32),
           "offsets": np_(b.offsets).view(np.uint32).astype(np.uint64),
           "total": int(np_(b.total)[0])}
    # the global key path first (its keys are checked too), then the binned
    # path the step uses; the raster runs on the binned lists
    br = Buffers(p.shape[1], sh, cams, device=dev, lists="radix")
    br.rec, br.rect, br.offsets, br.total = b.rec, b.rect, b.offsets, b.total
    br.intersections()
    torch.cuda.synchronize()
    K = br.K
    out["keys"] = np_(br.sorted_keys[:K]).view(np.uint64)
    out["vals"] = np_(br.sorted_vals[:K]).view(np.uint32)
    out["ranges"] = np_(br.ranges).view(np.uint32).reshape(-1, 2)
    out["overflow"] = int(np_(br.overflow)[0])
    out["radix_masks"] = np_(br.masks[:K]).view(np.uint16)  # gs_tile_masks on the sorted keys' lists
    del br
    # the binned builder on the sets of Gaussians each view sees
    bc = Buffers(p.shape[1], sh, cams, device=dev, lists="compact")
    bc.rec, bc.rect, bc.offsets, bc.total, bc.depth = b.rec, b.rect, b.offsets, b.total, b.depth
    bc.intersections()
    torch.cuda.synchronize()
    out["compact_vals"] = np_(bc.sorted_vals[:K]).view(np.uint32)
    out["compact_ranges"] = np_(bc.ranges).view(np.uint32).reshape(-1, 2)
    out["compact_masks"] = np_(bc.masks[:K]).view(np.uint16)
    out["compact_set_max"] = bc.set_max
    del bc
    b.intersections()
    b.rasterize(bg)
    torch.cuda.synchronize()
    out["binned_vals"] = np_(b.sorted_vals[:K]).view(np.uint32)
    out["binned_ranges"] = np_(b.ranges).view(np.uint32).reshape(-1, 2)
    out["binned_overflow"] = int(np_(b.overflow)[0])
    out["masks"] = np_(b.masks[:K]).view(np.uint16)
    out["image"] = np_(b.image)
    out["T_final"] = np_(b.T_final)
    out["n_contrib"] = np_(b.n_contrib)
    return b, out


def gpu_backward(b: Buffers, params_t: torch.Tensor, dL_np: np.ndarray, bg=(0.0, 0.0, 0.0)):
    b.dL.copy_(torch.from_numpy(np.ascontiguousarray(dL_np, dtype=np.float32)))
    grad = torch.empty_like(params_t)
    b.backward(params_t, grad, bg)
    torch.cuda.synchronize()
    g2 = np_(b.grad2d).reshape(b.V, b.n, L.GS_GRAD2D_ROWS)
    return g2, np_(grad)


def gpu_preprocess_bwd(b: Buffers, params_t: torch.Tensor, grad2d_np: np.ndarray):
    """Parameter gradients from a given [V][n][9] 2D gradient."""
    b.grad2d.copy_(torch.from_numpy(np.ascontiguousarray(grad2d_np, dtype=np.float32).reshape(-1)))
    grad = torch.empty_like(params_t)
    L.gs_preprocess_bwd(params_t, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, grad)
    torch.cuda.synchronize()
    return np_(grad)


def gpu_preprocess_bwd_adam(b: Buffers, params_t: torch.Tensor, grad2d_np: np.ndarray, m_np, v_np, lr, b1, b2, eps,
                            step, skip: int = 0):
    """The fused preprocess backward + Adam on a copy of the parameters:
    (parameters, m, v, gradient) after the call."""
    dev = b.device
    b.grad2d.copy_(torch.from_numpy(np.ascontiguousarray(grad2d_np, dtype=np.float32).reshape(-1)))
    th = params_t.clone()
    m, v = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (m_np, v_np))
    grad = torch.full_like(params_t, 7.0)
    flag = torch.full((1,), skip, dtype=torch.int32, device=dev)
    L.gs_preprocess_bwd_adam(th, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, m, v, lr, b1, b2, eps, step, skip=flag,
                             grad_params=grad)
    torch.cuda.synchronize()
    return np_(th), np_(m), np_(v), np_(grad)


def gpu_forward_l1(b: Buffers, target_np, bg=(0.0, 0.0, 0.0)):
    """The fused forward + L1 pass on the lists already in `b`: image, T_final,
    n_contrib, dL/dimage and the loss."""
    dev = b.device
    tgt = torch.from_numpy(np.ascontiguousarray(target_np, dtype=np.float32)).to(dev)
    b.rasterize_loss_l1(tgt, bg, image=True)
    torch.cuda.synchronize()
    return {"image": np_(b.image), "T_final": np_(b.T_final), "n_contrib": np_(b.n_contrib), "dL": np_(b.dL),
            "loss": float(np_(b.loss)[0])}


def gpu_fwd_bwd_l1(b: Buffers, target_np, bg=(0.0, 0.0, 0.0)):
    """The fused forward + L1 + backward pass on the lists already in `b`,
    with every optional output written."""
    dev = b.device
    tgt = torch.from_numpy(np.ascontiguousarray(target_np, dtype=np.float32)).to(dev)
    b.rasterize_fwd_bwd_l1(tgt, bg, outputs=True, image=True)
    torch.cuda.synchronize()
    return {"image": np_(b.image), "T_final": np_(b.T_final), "n_contrib": np_(b.n_contrib), "dL": np_(b.dL),
            "loss": float(np_(b.loss)[0]), "grad2d": np_(b.grad2d).reshape(b.V, b.n, L.GS_GRAD2D_ROWS).copy()}


def gpu_loss(image_np, target_np):
    dev = torch.device("cuda:0")
    img = torch.from_numpy(np.ascontiguousarray(image_np)).to(dev)
    tgt = torch.from_numpy(np.ascontiguousarray(target_np)).to(dev)
    dL = torch.empty_like(img)
    loss = torch.zeros(1, dtype=torch.float64, device=dev)
    V, _, H, W = img.shape
    L.gs_loss_l1(img, tgt, img.numel(), 1.0 / (3.0 * H * W * V), dL, loss)
    torch.cuda.synchronize()
    return float(np_(loss)[0]), np_(dL)


def gpu_adam(theta, g, m, v, lr, b1, b2, eps, step):
    dev = torch.device("cuda:0")
    ts = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (theta, g, m, v)]
    L.gs_adam_step(ts[0], ts[1], ts[2], ts[3], ts[0].numel(), lr, b1, b2, eps, step)
    torch.cuda.synchronize()
    return np_(ts[0]), np_(ts[2]), np_(ts[3])


# ---- comparisons --------------------------------------------------------------
def check_preprocess(gpu, orc):
    """Visibility, rectangles and counts exact; records to 1e-6 relative
    (their evaluation order is the same on both sides, so they are expected
    identical)."""
    iv = orc["iv"]
    vis_o = iv[..., O.INT_VIS] == 1
    rect_g = gpu["rect"]
    vis_g = (rect_g[..., 2] > rect_g[..., 0]) & (rect_g[..., 3] > rect_g[..., 1])
    assert np.array_equal(vis_o, vis_g), f"visibility differs at {np.argwhere(vis_o != vis_g)[:5]}"
    assert np.array_equal(rect_g[vis_o], iv[vis_o][:, O.INT_X0:O.INT_Y1 + 1])
    counts_o = np.where(vis_o, iv[..., O.INT_COUNT], 0).reshape(-1)
    off_o = O.exclusive_scan(counts_o.astype(np.uint32))
    assert gpu["total"] == int(off_o[-1])
    assert np.array_equal(gpu["offsets"], off_o & 0xffffffff)
    rg, ro = gpu["rec"][vis_o], orc["rec"][vis_o]
    pairs = [(L.REC_U, O.REC_U), (L.REC_V, O.REC_V), (L.REC_A, O.REC_CA), (L.REC_B, O.REC_CB),
             (L.REC_C, O.REC_CC), (L.REC_OPACITY, O.REC_O), (L.REC_R, 10), (L.REC_G, 11),
             (L.REC_BLUE, 12), (L.REC_DEPTH, O.REC_Z)]
    identical = 0
    for gi, oi in pairs:
        a, b = rg[:, gi].astype(np.float64), ro[:, oi].astype(np.float64)
        scale = np.maximum(np.abs(b), 1e-30)
        if gi in (L.REC_A, L.REC_B, L.REC_C):
            scale = np.maximum(np.abs(ro[:, O.REC_CA]), np.abs(ro[:, O.REC_CC])).astype(np.float64)
        if gi in (L.REC_R, L.REC_G, L.REC_BLUE):
            scale = np.maximum(scale, 1.0)
        rel = np.abs(a - b) / scale
        assert rel.max() <= 1e-6, (gi, rel.max())
        identical += int(np.sum(a == b))
    # depth bits drive the sort key: exact
    assert np.array_equal(rg[:, L.REC_DEPTH].view(np.uint32), ro[:, O.REC_Z].astype(np.float32).view(np.uint32))
    return {"visible": int(vis_o.sum()), "K": gpu["total"],
            "identical_fraction": identical / max(1, len(pairs) * rg.shape[0])}


def check_keys(gpu, cams):
    """The GPU's sorted keys / ids / ranges against the oracle's emit + library
    sort applied to the GPU's own rectangles and depths."""
    V = len(cams)
    rect = np.ascontiguousarray(gpu["rect"])
    vis = ((rect[..., 2] > rect[..., 0]) & (rect[..., 3] > rect[..., 1])).astype(np.uint8)
    z = np.ascontiguousarray(gpu["rec"][..., L.REC_DEPTH])
    keys, vals = O.emit_sorted(rect, vis, z, cams[0].tiles_x, cams[0].tiles_y)
    assert gpu["overflow"] == 0
    assert np.array_equal(gpu["keys"], keys), "sorted keys differ"
    assert np.array_equal(gpu["vals"], vals), "sorted ids differ"
    rng = O.tile_ranges(keys, V * cams[0].n_tiles)
    assert np.array_equal(gpu["ranges"], rng), "tile ranges differ"
    # the binned lists: the same ids and ranges
    assert gpu["binned_overflow"] == 0
    assert np.array_equal(gpu["binned_vals"], vals), "binned lists differ"
    assert np.array_equal(gpu["binned_ranges"], rng), "binned ranges differ"
    return keys.size


def check_masks(masks, vals, ranges, orc, cams, sample=None, seed=0, chunk=20000):
    """Sub-block masks of the list entries (gs_tile_masks): every pixel
    centre where the entry's alpha, in fp64 from the oracle's record, reaches
    1/255 with power <= 0 lies in a sub-block whose bit is set, and no bit is
    set for a sub-block outside the image. `sample` limits the entries
    checked (a seeded random subset). Returns the share of bits set."""
    V = len(cams)
    W, H = cams[0].width, cams[0].height
    TX, TY = (W + 15) // 16, (H + 15) // 16
    T = TX * TY
    K = len(vals)
    starts = ranges[:, 0].astype(np.int64)
    lens = (ranges[:, 1].astype(np.int64) - starts)
    tile_of = np.repeat(np.arange(V * T), lens)
    pos = np.concatenate([np.arange(s_, s_ + l_) for s_, l_ in zip(starts, lens) if l_ > 0]) if K else np.zeros(0, int)
    assert len(pos) == K
    idx = np.arange(K)
    if sample is not None and sample < K:
        idx = np.sort(np.random.default_rng(seed).choice(K, sample, replace=False))
    rec = orc["rec"].astype(np.float64)
    ii, jj = np.meshgrid(np.arange(16), np.arange(16))  # [j][i]
    sub = (jj // 4) * 4 + (ii // 4)
    bits_set = 0
    for c0 in range(0, len(idx), chunk):
        sel = idx[c0:c0 + chunk]
        p, tl = pos[sel], tile_of[sel]
        view, t = tl // T, tl % T
        tx, ty = t % TX, t // TX
        r = rec[view, vals[p].astype(np.int64)]
        m = masks[p].astype(np.int64)
        px = (tx * 16)[:, None, None] + ii[None] + 0.5
        py = (ty * 16)[:, None, None] + jj[None] + 0.5
        dx = r[:, 0, None, None] - px
        dy = r[:, 1, None, None] - py
        power = dx * (-0.5 * r[:, 6, None, None] * dx - r[:, 7, None, None] * dy) - 0.5 * r[:, 8, None, None] * dy * dy
        alpha = np.minimum(0.99, r[:, 9, None, None] * np.exp(np.minimum(power, 0.0)))
        inside = (px < W) & (py < H)
        need = inside & (power <= 0) & (alpha >= 1.0 / 255.0)
        bit = (m[:, None, None] >> sub[None]) & 1
        miss = need & (bit == 0)
        assert not miss.any(), f"{int(miss.any(axis=(1, 2)).sum())} entries miss a sub-block they reach"
        sbx = (tx * 16)[:, None] + 4 * np.arange(4)[None]
        sby = (ty * 16)[:, None] + 4 * np.arange(4)[None]
        outside = (sbx[:, None, :] >= W) | (sby[:, :, None] >= H)  # [entry][sy][sx]
        obits = (m[:, None, None] >> (4 * np.arange(4)[None, :, None] + np.arange(4)[None, None, :])) & 1
        assert not (outside & (obits == 1)).any(), "a bit is set for a sub-block outside the image"
        bits_set += int(sum(bin(int(x)).count("1") for x in m))
    return {"mask_bits_per_entry": bits_set / max(1, len(idx))}


def check_forward(gpu, fwd):
    amb = fwd["amb"] & 1
    ok = amb == 0
    # every output finite, ambiguous pixels included (a NaN fails every
    # comparison below, so the tests are written as "not within")
    for k in ("image", "T_final"):
        assert np.isfinite(gpu[k]).all(), f"non-finite {k} at {np.argwhere(~np.isfinite(gpu[k]))[:4]}"
    err = np.abs(gpu["image"] - fwd["image"]).max(axis=1)  # over channels
    bad = ok & ~(err <= IMAGE_ATOL)
    assert not bad.any(), f"{bad.sum()} unambiguous pixels off by up to {err[ok].max()}"
    nc_bad = ok & (gpu["n_contrib"] != fwd["n_contrib"])
    assert not nc_bad.any(), f"n_contrib differs at {nc_bad.sum()} unambiguous pixels"
    t_err = np.abs(gpu["T_final"] - fwd["T_final"])[ok]
    assert np.all(t_err <= IMAGE_ATOL), t_err.max()
    flipped = (~ok) & ((err > IMAGE_ATOL) | (gpu["n_contrib"] != fwd["n_contrib"]))
    return {"ambiguous": int(amb.sum()), "ambiguous_that_differ": int(flipped.sum()),
            "image_max_abs": float(err[ok].max(initial=0.0)), "T_max_abs": float(t_err.max(initial=0.0))}


def check_grad2d(g2_gpu, g2_ref, gabs):
    """g2_gpu and the oracle's, both [V][n][9]."""
    ref = g2_ref
    A = gabs
    err = np.abs(g2_gpu.astype(np.float64) - ref)
    lim = GRAD_RTOL * np.abs(ref) + GRAD_AFLOOR * A
    bad = ~(err <= lim)
    if bad.any():
        where = np.argwhere(bad)[:8]
        detail = [(tuple(int(x) for x in w), float(ref[tuple(w)]), float(g2_gpu[tuple(w)]), float(A[tuple(w)]))
                  for w in where]
        raise AssertionError(f"{bad.sum()} 2D gradients out of tolerance, worst {(err - lim).max()}; "
                             f"(index, ref, gpu, abs-sum): {detail}")
    nz = np.abs(ref) > 0
    within = np.mean(err[nz] <= GRAD_RTOL * np.abs(ref[nz])) if nz.any() else 1.0
    return {"grad2d_within_1e-3_rel": float(within)}


def check_param_grads(g_gpu, g_ref):
    ref = g_ref.astype(np.float64)
    row = np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(g_gpu.astype(np.float64) - ref)
    lim = PGRAD_RTOL * np.abs(ref) + PGRAD_ROWFLOOR * row
    bad = ~(err <= lim)
    assert not bad.any(), f"{bad.sum()} parameter gradients out of tolerance, rows {np.unique(np.nonzero(bad)[0])}"
    nz = np.abs(ref) > 0
    return {"pgrad_within_1e-3_rel": float(np.mean(err[nz] <= PGRAD_RTOL * np.abs(ref[nz]))) if nz.any() else 1.0}


def param_grads_e2e(g_gpu, g_ref):
    """End-to-end parameter gradients (each side from its own 2D gradients):
    the atomics' summation order makes cancelling sums differ in their last
    bits, so this reports the share of significant entries (above 1e-3 of
    their row's largest) within 1e-3 relative."""
    ref = g_ref.astype(np.float64)
    row = np.abs(ref).max(axis=1, keepdims=True)
    sig = np.abs(ref) > 1e-3 * row
    err = np.abs(g_gpu.astype(np.float64) - ref)
    ok = err <= 1e-3 * np.abs(ref)
    return {"e2e_within_1e-3_rel_of_significant": float(ok[sig].mean()) if sig.any() else 1.0,
            "e2e_within_1e-3_rel_all_nonzero": float(ok[ref != 0].mean()) if (ref != 0).any() else 1.0}


def check_adam(gpu, ref, theta0, g, m0, lr, b1):
    th_g, m_g, v_g = gpu
    th_r, m_r, v_r = ref
    f64 = lambda a: np.asarray(a, np.float64)
    assert np.all(np.abs(f64(th_g) - th_r) <= ADAM_RTOL * (np.abs(f64(th_r)) + lr))
    assert np.all(np.abs(f64(m_g) - m_r) <= ADAM_RTOL * (np.abs(b1 * f64(m0)) + np.abs((1 - b1) * f64(g))) + 1e-30)
    assert np.all(np.abs(f64(v_g) - v_r) <= ADAM_RTOL * np.abs(f64(v_r)) + 1e-38)
