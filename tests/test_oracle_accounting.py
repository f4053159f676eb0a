"""Per-Gaussian storage accounting against the figures the pages print
(tests/golden/accounting.json, each entry cited)."""

import json
import os

import pytest

from gaussian_splatting_differentiable_ewa_amd.scenes import CONFIGS, param_rows

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting.json")))


def test_param_rows_match_page_breakdown():
    parts = GOLD["params_per_gaussian_sh3"]["parts"]
    assert sum(parts.values()) == GOLD["params_per_gaussian_sh3"]["value"] == param_rows(3)
    # SH block = 3 colour channels x (d+1)^2 coefficients
    assert parts["sh"] == 3 * (3 + 1) ** 2
    assert param_rows(0) == 14


def test_bytes_per_gaussian_with_adam():
    # fp32 parameters plus the two Adam moments of the same shape
    assert param_rows(3) * 4 * 3 == GOLD["bytes_per_gaussian_with_adam_sh3"]["value"]


def test_storage_per_million_and_largest_run():
    b = param_rows(3) * 4
    assert b * 1e6 / 1e9 == pytest.approx(GOLD["param_bytes_per_million_gb"]["value"])
    run = GOLD["largest_run"]
    assert b * run["gaussians"] / 1e9 == pytest.approx(run["bytes_gb"], abs=5e-4)


def test_mi300x_capacity():
    cap = GOLD["mi300x_capacity"]
    n = cap["hbm_gb"] * 1e9 / GOLD["bytes_per_gaussian_with_adam_sh3"]["value"]
    assert round(n / 1e6) == cap["gaussians_millions_approx"]


def test_city_block_state_bytes():
    cfg = CONFIGS[4]
    assert cfg.P * 4 * 3 * cfg.n / 1e9 == pytest.approx(28.32)
