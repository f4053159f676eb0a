"""The GPU side of the oracle's near-threshold band: the raster passes' exp
(gs_raster_exp) at every fp32 power in [-5.6, 0] lies within the band the
oracle flags decisions with (or_exp_band, relative to the oracle's expf), and
the hardware exp2 is within the one ulp of 2^fl(p log2 e) the band assumes."""

import numpy as np
import pytest

from tests.test_oracle_band import LOG2E_F32, _powers_by_binade

pytestmark = pytest.mark.gpu


def test_exp_path_within_oracle_band(oracle_lib):
    import torch

    from gaussian_splatting_differentiable_ewa_amd import _lib as L

    O = oracle_lib
    dev = torch.device("cuda:0")
    worst_band = 0.0  # max over powers of |G_gpu / G_oracle - 1| / band
    worst_ulp = 0.0  # max error of the hardware exp2 against 2^y, in ulps of the result
    n = 0
    for p in _powers_by_binade():
        x = torch.from_numpy(p).to(dev)
        y = torch.empty_like(x)
        L.gs_raster_exp(x, y)
        g = y.cpu().numpy().astype(np.float64)
        n += p.size
        ratio = np.abs(g / O.expf(p).astype(np.float64) - 1.0) / O.exp_band(p)
        worst_band = max(worst_band, float(ratio.max()))
        two_y = np.exp2((p * LOG2E_F32).astype(np.float64))
        ulp = np.spacing(two_y.astype(np.float32)).astype(np.float64)
        worst_ulp = max(worst_ulp, float((np.abs(g - two_y) / ulp).max()))
    print({"powers": n, "max_over_band": worst_band, "hw_exp2_max_ulp": worst_ulp})
    assert worst_ulp <= O.lib().or_exp_hw_ulp()
    assert worst_band <= 1.0
