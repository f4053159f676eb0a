"""One training step on one GPU through the C ABI.

PyTorch only allocates device memory and provides the stream; every stage is a
call into the HIP library (``_lib``). The only device-to-host transfer per step
is the intersection count K, read after ``gs_preprocess`` to size the list
buffers (they are kept and only grown).

The per-tile lists come from ``gs_tile_lists`` (binning, then a sort of each
tile on its own) or from the global 64-bit key path (``gs_emit_intersections``,
``gs_sort_keys``, ``gs_tile_ranges``); both give the same ids and ranges.
``lists="auto"`` picks binning unless the (view, Gaussian) pairs outnumber the
intersections (a large scene mostly outside the views, where binning's two
passes over every pair cost more than the sort).
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import _lib as L


class Buffers:
    """Device buffers of one step for N Gaussians and a set of same-size views."""

    def __init__(self, n: int, sh_degree: int, cams: Sequence, device="cuda", lists: str = "auto"):
        if lists not in ("auto", "binned", "radix"):
            raise ValueError(f"unknown list builder {lists!r}")
        self.lists = lists
        self.path = "binned" if lists == "auto" else lists
        self.n = int(n)
        self.sh_degree = int(sh_degree)
        self.cams = list(cams)
        self.V = len(cams)
        self.W, self.H = cams[0].width, cams[0].height
        self.TX = (self.W + L.GS_TILE - 1) // L.GS_TILE
        self.TY = (self.H + L.GS_TILE - 1) // L.GS_TILE
        self.T = self.TX * self.TY
        self.P = L.param_rows(sh_degree)
        V, n, dev = self.V, self.n, device
        self.rec = torch.empty(V * n * L.GS_REC_FLOATS, dtype=torch.float32, device=dev)
        self.rect = torch.empty(V * n * 4, dtype=torch.int16, device=dev)
        self.offsets = torch.empty(V * n + 1, dtype=torch.int32, device=dev)
        self.total = torch.zeros(1, dtype=torch.int64, device=dev)
        self.pre_ws = torch.empty(L.preprocess_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
        self.ranges = torch.empty(V * self.T * 2, dtype=torch.int32, device=dev)
        self.image = torch.empty(V, 3, self.H, self.W, dtype=torch.float32, device=dev)
        self.T_final = torch.empty(V, self.H, self.W, dtype=torch.float32, device=dev)
        self.n_contrib = torch.empty(V, self.H, self.W, dtype=torch.int32, device=dev)
        self.dL = torch.empty_like(self.image)
        self.loss = torch.zeros(1, dtype=torch.float64, device=dev)
        self.grad2d = torch.empty(V * L.GS_GRAD2D_ROWS * n, dtype=torch.float32, device=dev)
        self.overflow = torch.zeros(1, dtype=torch.int32, device=dev)
        self.fwd_l1_ws = torch.empty(L.rasterize_fwd_l1_workspace_bytes(V, self.W, self.H), dtype=torch.uint8,
                                     device=dev)
        self.end_bit = L.sort_end_bit(V, self.T)
        self.capacity = 0
        self.allocated_for = None
        self.K = 0
        self.sorted_in_alt = False
        self.device = dev

    def ensure_capacity(self, K: int, slack: float = 1.25):
        if K <= self.capacity and self.capacity > 0 and self.allocated_for == self.path:
            return
        cap = max(int(K * slack) + 4096, self.capacity)
        dev = self.device
        self.vals = torch.empty(cap, dtype=torch.int32, device=dev)
        self.allocated_for = self.path
        if self.path == "radix":
            self.keys = torch.empty(cap, dtype=torch.int64, device=dev)
            self.keys_alt = torch.empty(cap, dtype=torch.int64, device=dev)
            self.vals_alt = torch.empty(cap, dtype=torch.int32, device=dev)
            self.sort_ws = torch.empty(L.sort_workspace_bytes(cap), dtype=torch.uint8, device=dev)
        else:
            self.tl_ws = torch.empty(L.tile_lists_workspace_bytes(self.n, self.V, self.W, self.H, cap), dtype=torch.uint8,
                                     device=dev)
        self.capacity = cap

    def workspace_bytes(self) -> int:
        """Bytes of the intersection lists and their workspaces."""
        if self.capacity == 0:
            return 0
        if self.path == "radix":
            return 2 * 12 * self.capacity + self.sort_ws.numel()
        return 4 * self.capacity + self.tl_ws.numel()

    @property
    def sorted_keys(self):
        return self.keys_alt if self.sorted_in_alt else self.keys

    @property
    def sorted_vals(self):
        return self.vals_alt if self.sorted_in_alt else self.vals

    # ---- stages ------------------------------------------------------------
    def preprocess(self, params):
        L.gs_preprocess(params, self.n, self.sh_degree, self.cams, self.rec, self.rect, self.offsets,
                        self.total, self.pre_ws)

    def intersections(self):
        """Read K, then build the per-tile lists and their ranges."""
        self.K = int(self.total.item())
        if self.K >= 2 ** 32:
            raise L.GsError(f"{self.K} intersections exceed the 32-bit key index")
        if self.lists == "auto":
            self.path = "binned" if self.V * self.n <= self.K else "radix"
        self.ensure_capacity(self.K)
        if self.path == "binned":
            self.sorted_in_alt = False
            L.gs_tile_lists(self.rec, self.rect, self.n, self.V, self.W, self.H, self.vals, self.capacity,
                            self.ranges, self.overflow, self.tl_ws)
            return
        L.gs_emit_intersections(self.rec, self.rect, self.offsets, self.n, self.V, self.W, self.H,
                                self.keys, self.vals, self.capacity, self.overflow)
        self.sorted_in_alt = L.gs_sort_keys(self.keys, self.vals, self.keys_alt, self.vals_alt, self.K,
                                            self.end_bit, self.sort_ws)
        L.gs_tile_ranges(self.sorted_keys, self.K, self.V * self.T, self.ranges)

    def rasterize(self, bg=(0.0, 0.0, 0.0)):
        L.gs_rasterize_fwd(self.rec, self.n, self.ranges, self.sorted_vals, self.cams, bg, self.image,
                           self.T_final, self.n_contrib)

    def loss_l1(self, target):
        scale = 1.0 / (3.0 * self.H * self.W * self.V)
        L.gs_loss_l1(self.image, target, self.image.numel(), scale, self.dL, self.loss)

    def rasterize_loss_l1(self, target, bg=(0.0, 0.0, 0.0), image: bool = False):
        """Forward raster and L1 loss in one pass; the image is written only
        when asked for."""
        scale = 1.0 / (3.0 * self.H * self.W * self.V)
        L.gs_rasterize_fwd_l1(self.rec, self.n, self.ranges, self.sorted_vals, self.cams, bg, target, scale,
                              self.image if image else None, self.T_final, self.n_contrib, self.dL, self.loss,
                              self.fwd_l1_ws)

    def backward(self, params, grad, bg=(0.0, 0.0, 0.0)):
        L.gs_rasterize_bwd(self.rec, self.n, self.ranges, self.sorted_vals, self.cams, bg, self.T_final,
                           self.n_contrib, self.dL, self.grad2d)
        L.gs_preprocess_bwd(params, self.n, self.sh_degree, self.cams, self.rect, self.grad2d, grad)


def render(params: torch.Tensor, sh_degree: int, cams: Sequence, bg=(0.0, 0.0, 0.0)) -> torch.Tensor:
    """Forward render of ``params`` through ``cams``; returns [V][3][H][W]."""
    b = Buffers(params.shape[1], sh_degree, cams, device=params.device)
    b.preprocess(params)
    b.intersections()
    b.rasterize(bg)
    return b.image


class TrainStep:
    """Parameters, Adam state and buffers of fwd + L1 + bwd + Adam steps."""

    def __init__(self, params: torch.Tensor, sh_degree: int, cams: Sequence, target: torch.Tensor,
                 lr=1e-3, betas=(0.9, 0.999), eps=1e-15, bg=(0.0, 0.0, 0.0),
                 m: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None):
        assert params.is_cuda and params.dtype == torch.float32 and params.is_contiguous()
        self.params = params
        self.sh_degree = sh_degree
        self.buf = Buffers(params.shape[1], sh_degree, cams, device=params.device)
        assert params.shape[0] == self.buf.P
        self.target = target.contiguous()
        self.m = torch.zeros_like(params) if m is None else m
        self.v = torch.zeros_like(params) if v is None else v
        self.grad = torch.empty_like(params)
        self.lr, self.betas, self.eps, self.bg = lr, betas, eps, bg
        self.t = 0

    def step(self):
        b = self.buf
        self.t += 1
        b.preprocess(self.params)
        b.intersections()
        b.rasterize_loss_l1(self.target, self.bg)
        b.backward(self.params, self.grad, self.bg)
        L.gs_adam_step(self.params, self.grad, self.m, self.v, self.params.numel(), self.lr, self.betas[0],
                       self.betas[1], self.eps, self.t)
