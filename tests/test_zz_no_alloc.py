"""gs_rasterize_fwd_bwd_l1_noalloc (the fused raster pass on the library's
fixed per-device workspace, for callers that cannot allocate) against
gs_rasterize_fwd_bwd_l1 with a caller-owned workspace, through the C ABI, on
two calls in a row: the 4-view 1080p headline lists, then the smaller
two-view 250x190 scene's (the second call reuses the array the first left
filled). Image, T_final, n_contrib and dL/dimage bit for bit (the same
kernels on the same inputs); the loss and the 2D gradients equal up to the
order of their atomic additions; and both against the oracle's L1 of that
image."""

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import _lib as L
from gaussian_splatting_differentiable_ewa_amd import scenes as S
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _lists(cfg, n=None):
    import torch

    from gaussian_splatting_differentiable_ewa_amd.step import Buffers

    dev = torch.device("cuda:0")
    cams = cfg.cameras()
    p = torch.from_numpy(S.make_params(cfg, n=n)).to(dev)
    b = Buffers(p.shape[1], cfg.sh_degree, cams, device=dev)
    b.preprocess(p)
    b.intersections()
    target = torch.from_numpy(S.random_image(cfg.target_seed, len(cams), cams[0].height, cams[0].width)).to(dev)
    return b, target


def _run(b, target, noalloc):
    import torch
    dev = b.device
    out = {k: torch.full_like(getattr(b, k), -7) for k in ("image", "T_final", "n_contrib", "dL")}
    loss = torch.full((1,), 5.0, dtype=torch.float64, device=dev)
    g2 = torch.full_like(b.grad2d, 3.0)
    scale = 1.0 / (3.0 * b.H * b.W * b.V)
    kw = dict(image=out["image"], T_final=out["T_final"], n_contrib=out["n_contrib"], dL_dimage=out["dL"])
    if noalloc:
        L.gs_rasterize_fwd_bwd_l1_noalloc(b.rec, b.n, b.ranges, b.sorted_vals, b.masks, b.cams, (0.0, 0.0, 0.0),
                                          target, scale, loss, g2, **kw)
    else:
        L.gs_rasterize_fwd_bwd_l1(b.rec, b.n, b.ranges, b.sorted_vals, b.masks, b.cams, (0.0, 0.0, 0.0), target,
                                  scale, loss, g2, b.fwd_l1_ws, **kw)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["loss"] = float(loss.item())
    res["grad2d"] = g2.view(b.V, b.n, 9).double().cpu().numpy()
    return res


@pytest.mark.parametrize("calls", [[S.CONFIGS[2], S.RAGGED]], ids=["headline-then-ragged"])
def test_noalloc_equals_workspace_form(calls):
    for k, cfg in enumerate(calls):
        b, target = _lists(cfg)
        print(f"[noalloc] call {k + 1}: {cfg.name}, {b.V * b.T} tiles", flush=True)
        ref = _run(b, target, noalloc=False)
        got = _run(b, target, noalloc=True)
        for key in ("image", "T_final", "n_contrib", "dL"):
            assert np.array_equal(got[key], ref[key]), key
        assert got["loss"] == pytest.approx(ref["loss"], rel=1e-12)  # fp64 atomics, order varies
        loss_o, dL_o = O.loss_l1(ref["image"], target.cpu().numpy())
        assert np.array_equal(ref["dL"], dL_o)
        assert ref["loss"] == pytest.approx(loss_o, rel=1e-6)
        a, c = ref["grad2d"], got["grad2d"]
        scale = np.abs(a).max()
        assert np.all(np.abs(a - c) <= 1e-4 * np.abs(a) + 1e-7 * scale)
        del b
