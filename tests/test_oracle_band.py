"""Pins of the oracle's near-threshold band: the pixels whose alpha >= 1/255,
0.99-clamp or T' < 1e-4 decisions a GPU's exp() may take the other way, which
the parity tests exclude from element-wise comparison.

The band (gs_oracle.c, or_exp_band) is derived, not chosen: the GPU's raster
passes take exp(p) as a hardware 2^y of y = fl(p * fl32(log2 e)), the oracle
the C library's expf. These tests check

* the C library's expf against fp64 exp at every fp32 power in [-5.6, 0]
  (alpha >= 1/255 needs exp(p) >= 1/255, p >= ln(1/255) = -5.54);
* that the band covers, at every fp32 power there, the exact error of the
  GPU's argument (fp64 evaluation of 2^fl(p L) against e^p) combined with one
  ulp of the hardware exp2 and the library's measured error at that power,
  and that it is at most five times that bound (its closed form rounds the
  argument's error up to a whole ulp of y and the library's to its maximum);
* that every decision an exp anywhere inside the band changes is flagged: the
  oracle's render with each exp moved to an edge of its band flips only
  flagged pixels, while a band cut to a quarter misses some.
"""

import math

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import scenes as S

P_LO = -5.6  # below ln(1/255): alpha < 1/255 whatever the opacity
U = 2.0 ** -24
LOG2E_F32 = np.float32(1.4426950408889634)


def _powers_by_binade():
    """Every fp32 power in [P_LO, -2^-30], one binade (or the part of it in
    range) at a time, plus 0 and a few tiny and subnormal values."""
    yield np.array([0.0, -0.0, -1e-40, -1e-38, -2.0 ** -40, -2.0 ** -31], dtype=np.float32)
    for e in range(-30, 3):
        lo = np.float32(2.0 ** e).view(np.uint32)
        hi = np.float32(min(2.0 ** (e + 1), -P_LO)).view(np.uint32)
        bits = np.arange(lo, hi + (1 if 2.0 ** (e + 1) > -P_LO else 0), dtype=np.uint32)
        yield -bits.view(np.float32)


def test_band_constants_are_its_derivation(oracle_lib):
    L = oracle_lib.lib()
    assert L.or_exp_hw_ulp() == 1.0
    assert L.or_exp_libm_rel() == pytest.approx(1.01 * U, rel=1e-12)
    # rG at p = 0: only the hardware's ulp and the library's error remain
    assert L.or_exp_band(0.0) == pytest.approx((1 + 2 * U) / (1 - 1.01 * U) - 1, rel=1e-9)
    # the product o G adds one rounding on each side
    for p in (0.0, -1.0, -5.5):
        rg = L.or_exp_band(p)
        assert L.or_alpha_band(p) == pytest.approx((1 + rg) * (1 + U) / (1 - U) - 1, rel=1e-9)
    # at the far end of the range the argument's rounding dominates: about
    # ln 2 * 5.5 * (|L - log2 e| + L 2^-24) ~ 4.0e-7 on top of 1.8e-7
    assert 5.5e-7 < L.or_exp_band(-5.5) < 6.0e-7


@pytest.mark.slow
def test_libm_expf_and_band_cover_exact_error(oracle_lib):
    O = oracle_lib
    libm_rel = O.lib().or_exp_libm_rel()
    hw = O.lib().or_exp_hw_ulp() * 2.0 * U
    worst_libm = 0.0
    worst_ratio_hi = 0.0
    worst_cover = math.inf
    n = 0
    for p in _powers_by_binade():
        n += p.size
        p64 = p.astype(np.float64)
        e = np.exp(p64)
        # the C library's expf against fp64 (fp64's own error is ~1e-16)
        libm = np.abs(O.expf(p).astype(np.float64) / e - 1.0)
        worst_libm = max(worst_libm, float(libm.max()))
        # the GPU's argument, exactly: y = fl32(p * fl32(log2 e)), 2^y in fp64
        y = (p * LOG2E_F32).astype(np.float64)
        arg = np.abs(np.exp2(y) / e - 1.0)
        exact = (1.0 + arg) * (1.0 + hw) / (1.0 - libm) - 1.0
        band = O.exp_band(p)
        worst_cover = min(worst_cover, float((band / exact).min()))
        worst_ratio_hi = max(worst_ratio_hi, float((band / exact).max()))
    print({"powers": n, "libm_max_rel": worst_libm, "libm_bound": libm_rel,
           "band_over_exact_min": worst_cover, "band_over_exact_max": worst_ratio_hi})
    assert n > 2.5e8
    assert worst_libm <= libm_rel
    assert worst_cover >= 1.0, "the band misses the exact error at some power"
    assert worst_ratio_hi <= 5.0, "the band is more than five times the exact error somewhere"


def _scene(cfg_id):
    cfg = S.CONFIGS[cfg_id]
    return cfg, S.make_params(cfg), cfg.cameras()


@pytest.mark.parametrize("cfg_id", [0, 1], ids=["tiny", "object"])
def test_flags_cover_every_flip_within_the_band(oracle_lib, cfg_id):
    """Each exp moved to either edge of its band (or the edge picked per
    power): every pixel whose decisions change is flagged, and every pixel
    whose image (beyond 1e-4) or n_contrib changes has the image flag."""
    O = oracle_lib
    cfg, params, cams = _scene(cfg_id)
    proj = O.preprocess(params, cfg.sh_degree, cams)
    ref = O.render_fwd(proj, cams)
    amb = ref["amb"]
    flips = 0
    for mode in (1, -1, 2):
        with O.exp_perturbed(mode):
            f = O.render_fwd(proj, cams)
        sig = f["sig"] != ref["sig"]
        img = (np.abs(f["image"] - ref["image"]).max(axis=1) > 1e-4) | (f["n_contrib"] != ref["n_contrib"])
        assert not (sig & (amb == 0)).any(), f"mode {mode}: {int((sig & (amb == 0)).sum())} unflagged flips"
        assert not (img & ((amb & 1) == 0)).any()
        flips += int(sig.sum())
    n_px = amb.size
    print({"scene": cfg.name, "flagged": int((amb != 0).sum()), "image_flagged": int((amb & 1).sum()),
           "flips_over_3_runs": flips, "pixels": n_px})
    # the band is narrow: at most 0.02 % of the pixels
    assert int((amb & 1).sum()) <= max(16, n_px // 5000)


def test_narrowed_band_misses_flips(oracle_lib):
    """The check above has teeth: with the flags' band cut to a quarter, an
    exp at the edge of the true band flips pixels the flags miss."""
    O = oracle_lib
    cfg, params, cams = _scene(1)
    proj = O.preprocess(params, cfg.sh_degree, cams)
    with O.band_scaled(0.25):
        ref = O.render_fwd(proj, cams)
    missed = 0
    for mode in (1, 2):
        with O.exp_perturbed(mode):
            f = O.render_fwd(proj, cams)
        missed += int(((f["sig"] != ref["sig"]) & (ref["amb"] == 0)).sum())
    assert missed > 0
