"""gs_sort_keys through the C ABI against a stable library sort (numpy's
stable argsort on the masked keys) on adversarial inputs: sizes around the
4096-key tile and the 64-lane wave, heavy key repetition (stability), every
digit varying, and pass counts from 1 to 8."""

import numpy as np
import pytest

from gaussian_splatting_differentiable_ewa_amd import _lib as L

pytestmark = pytest.mark.gpu

CASES = [
    # (n, end_bit, key kind)
    (1, 8, "random"), (63, 13, "random"), (64, 47, "random"), (4095, 47, "random"), (4096, 40, "random"),
    (4097, 47, "few"), (100_003, 64, "random"), (100_003, 47, "few"), (250_000, 47, "tiles"),
    (1_000_001, 33, "same"), (2_000_000, 47, "tiles"),
]


def _keys(rng, n, end_bit, kind):
    if kind == "random":
        k = rng.integers(0, 2 ** 63, n, dtype=np.int64).astype(np.uint64) << np.uint64(1)
        k |= rng.integers(0, 2, n, dtype=np.int64).astype(np.uint64)
    elif kind == "few":  # many equal keys: stability decides the order
        k = rng.integers(0, 7, n, dtype=np.int64).astype(np.uint64) * np.uint64(0x0101010101010101)
    elif kind == "same":
        k = np.full(n, 0x12345678, dtype=np.uint64)
    else:  # the intersection key: (tile << 32) | positive float depth bits
        tile = rng.integers(0, 32640, n, dtype=np.int64).astype(np.uint64)
        z = rng.uniform(4.0, 40.0, n).astype(np.float32).view(np.uint32).astype(np.uint64)
        k = (tile << np.uint64(32)) | z
    if end_bit < 64:
        k &= np.uint64((1 << end_bit) - 1)
    return k


@pytest.mark.parametrize("n,end_bit,kind", CASES)
def test_sort_matches_stable_sort(n, end_bit, kind):
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(n + end_bit)
    keys = _keys(rng, n, end_bit, kind)
    vals = np.arange(n, dtype=np.uint32)
    order = np.argsort(keys, kind="stable")
    kt = torch.from_numpy(keys.view(np.int64).copy()).to(dev)
    vt = torch.from_numpy(vals.view(np.int32).copy()).to(dev)
    ka, va = torch.empty_like(kt), torch.empty_like(vt)
    ws = torch.empty(L.sort_workspace_bytes(n), dtype=torch.uint8, device=dev)
    for _ in range(2):  # a second call on the same workspace starts from a clean state
        kt2, vt2 = kt.clone(), vt.clone()
        alt = L.gs_sort_keys(kt2, vt2, ka, va, n, end_bit, ws)
        torch.cuda.synchronize()
        ko = (ka if alt else kt2).cpu().numpy().view(np.uint64)
        vo = (va if alt else vt2).cpu().numpy().view(np.uint32)
        assert np.array_equal(ko, keys[order])
        assert np.array_equal(vo, vals[order])
