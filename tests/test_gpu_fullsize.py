"""GPU parity at the full sizes of the three large scenes, through the same
Buffers/launches the benchmark times:

  * headline: 1M Gaussians, SH 3, four 1920x1080 views;
  * stress:   5M Gaussians, SH 3, one 3840x2160 view;
  * city:     40M Gaussians, SH 3, one 1920x1080 view, far plane 120.

Every pixel and every visible Gaussian is compared (the oracle is cheap enough
per pixel); parameter gradients are compared on a seeded sample of Gaussians
(the chain rule is per Gaussian, so a sample is compared exactly), Adam on a
seeded sample of elements of the full-size update. The L1 target is a seeded
uniform image: rendering a target scene would cost a second oracle render and
adds nothing to what is checked."""

import time

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import scenes as S
from oracle import oracle as O
from tests import parity as PY

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SAMPLE_VISIBLE = 60_000
SAMPLE_HIDDEN = 10_000


def _log(msg):
    print(f"[fullsize] {msg}", flush=True)


@pytest.fixture(scope="module", params=[2, 3, 4], ids=["headline", "stress", "city"])
def run(request):
    import torch
    assert torch.cuda.is_available()
    cfg = S.CONFIGS[request.param]
    cams = cfg.cameras()
    t0 = time.time()
    _log(f"scene {cfg.name}: drawing {cfg.n} Gaussians")
    params = S.make_params(cfg)
    _log(f"params ready ({time.time() - t0:.1f}s); oracle preprocess + forward")
    orc = O.preprocess(params, cfg.sh_degree, cams)
    fwd = O.render_fwd(orc, cams)
    _log(f"oracle forward done ({time.time() - t0:.1f}s); GPU forward")
    b, gpu = PY.gpu_forward(params, cfg.sh_degree, cams)
    target = S.random_image(cfg.target_seed, len(cams), cams[0].height, cams[0].width)
    _log(f"GPU forward done ({time.time() - t0:.1f}s), K = {gpu['total']}")
    yield {"cfg": cfg, "params": params, "cams": cams, "orc": orc, "fwd": fwd, "buf": b, "gpu": gpu,
           "target": target}
    del b
    torch.cuda.empty_cache()


def test_preprocess(run):
    st = PY.check_preprocess(run["gpu"], run["orc"])
    _log(st)
    assert st["K"] > 0


def test_keys_sort_ranges(run):
    K = PY.check_keys(run["gpu"], run["cams"])
    ranges = run["gpu"]["ranges"]
    per_tile = ranges[:, 1].astype(np.int64) - ranges[:, 0]
    _log({"K": K, "K_per_gaussian": K / run["cfg"].n, "max_per_tile": int(per_tile.max())})


def test_forward(run):
    st = PY.check_forward(run["gpu"], run["fwd"])
    _log(st)
    n_px = run["fwd"]["image"][:, 0].size
    assert st["ambiguous"] <= max(16, n_px // 5000)


def _dL(run):
    fwd = run["fwd"]
    _, dL = O.loss_l1(fwd["image"], run["target"])
    dL[np.broadcast_to((fwd["amb"] != 0)[:, None], dL.shape)] = 0
    return dL


def test_loss(run):
    loss_o, dL_o = O.loss_l1(run["gpu"]["image"], run["target"])
    loss_g, dL_g = PY.gpu_loss(run["gpu"]["image"], run["target"])
    assert loss_g == pytest.approx(loss_o, rel=1e-6)
    assert np.array_equal(dL_g, dL_o)
    # the fused forward + L1 pass the step uses
    fused = PY.gpu_forward_l1(run["buf"], run["target"])
    assert np.array_equal(fused["image"], run["gpu"]["image"])
    assert np.array_equal(fused["dL"], dL_o)
    assert fused["loss"] == pytest.approx(loss_o, rel=1e-6)


def test_backward_and_adam(run):
    cfg, params, cams = run["cfg"], run["params"], run["cams"]
    dL = _dL(run)
    t0 = time.time()
    g2_ref, gabs = O.render_bwd(run["orc"], cams, dL, with_abs=True)
    _log(f"oracle backward done ({time.time() - t0:.1f}s)")
    g2_gpu, grad_gpu = PY.gpu_backward(run["buf"], run["gpu"]["params_t"], dL)
    vis = run["orc"]["iv"][..., O.INT_VIS] == 1  # [V][N]
    # hidden (view, Gaussian) pairs receive exactly zero
    assert not np.any(g2_gpu[~vis]), "a culled Gaussian received a 2D gradient"
    st = PY.check_grad2d(g2_gpu[vis], g2_ref[vis], gabs[vis])
    _log(st)
    del gabs

    # parameter gradients on a seeded sample: stage-wise (the GPU's 2D
    # gradients on both sides) and end to end (each side's own)
    rng = np.random.default_rng(1234)
    any_vis = np.nonzero(vis.any(axis=0))[0]
    hidden = np.nonzero(~vis.any(axis=0))[0]
    idx = np.concatenate([rng.choice(any_vis, min(SAMPLE_VISIBLE, any_vis.size), replace=False),
                          rng.choice(hidden, min(SAMPLE_HIDDEN, hidden.size), replace=False)])
    idx.sort()
    sub = np.ascontiguousarray(params[:, idx])
    g_ref = O.preprocess_bwd(sub, cfg.sh_degree, cams, np.ascontiguousarray(g2_gpu[:, idx]).astype(np.float64))
    st = PY.check_param_grads(grad_gpu[:, idx], g_ref)
    _log(st)
    g_e2e = O.preprocess_bwd(sub, cfg.sh_degree, cams, np.ascontiguousarray(g2_ref[:, idx]))
    st = PY.param_grads_e2e(grad_gpu[:, idx], g_e2e)
    _log(st)
    assert st["e2e_within_1e-3_rel_of_significant"] > 0.999
    del g2_ref, g2_gpu

    # Adam, first step from zero moments, over all P x N elements on the GPU;
    # a seeded sample of elements is compared with the oracle's update
    import torch
    dev = torch.device("cuda:0")
    th = run["gpu"]["params_t"].clone()
    g = torch.from_numpy(grad_gpu).to(dev)
    m = torch.zeros_like(th)
    v = torch.zeros_like(th)
    PY.L.gs_adam_step(th, g, m, v, th.numel(), cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, 1)
    torch.cuda.synchronize()
    flat = np.unique(rng.integers(0, th.numel(), 200_000))
    fi = torch.from_numpy(flat).to(dev)
    out = [PY.np_(x.reshape(-1)[fi]) for x in (th, m, v)]
    g_s = grad_gpu.reshape(-1)[flat]
    z = np.zeros_like(g_s)
    ref = O.adam(params.reshape(-1)[flat], g_s, z, z, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, 1)
    PY.check_adam(out, ref, params.reshape(-1)[flat], g_s, z, cfg.lr, cfg.beta1)
    # untouched elements (zero gradient, zero moments) stay bit-identical
    zero_g = g_s == 0
    assert np.array_equal(out[0][zero_g], params.reshape(-1)[flat][zero_g])
