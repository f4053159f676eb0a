"""One training step on one GPU through the C ABI.

PyTorch only allocates device memory and provides the stream; every stage is a
call into the HIP library (``_lib``). The intersection count K sizes the list
buffers (kept, and only grown). ``Buffers.intersections`` reads it on the host
after ``gs_preprocess``; ``TrainStep`` does so only when it must (the first
step, the global-sort builder), and otherwise builds the lists with the
capacity it has and lets the device guard the update: the lists' overflow flag
is folded into a sticky flag, Adam is skipped while it is set, and K and the
flag are copied back without waiting. When a copied flag shows an overflow,
the steps from that one on are redone with larger buffers (their updates were
skipped, so the state is exactly that of the step before).

The per-tile lists come from ``gs_tile_lists`` (binning, then a sort of each
tile on its own) or from the global 64-bit key path (``gs_emit_intersections``,
``gs_sort_keys``, ``gs_tile_ranges``); all give the same ids and ranges.
``lists="compact"`` bins only the Gaussians each view sees: ``gs_window_gaussians``
over the whole image lists them, and ``gs_tile_lists`` bins that set with its
grid sized for it (planned from the set sizes read when K is read).
``lists="auto"`` picks binning of every pair unless the (view, Gaussian) pairs
outnumber the intersections (a large scene mostly outside the views), and the
compacted set then.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import _lib as L


class Buffers:
    """Device buffers of one step for N Gaussians and a set of same-size views."""

    def __init__(self, n: int, sh_degree: int, cams: Sequence, device="cuda", lists: str = "auto",
                 offsets: Optional[bool] = None):
        if lists not in ("auto", "binned", "radix", "compact"):
            raise ValueError(f"unknown list builder {lists!r}")
        self.lists = lists
        # the per-entry offsets of the tile counts: only the global key sort
        # needs them (the preprocess then scans the counts; otherwise it forms
        # the total alone)
        self.with_offsets = lists == "radix" if offsets is None else bool(offsets)
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
        self.depth = torch.empty(V * n, dtype=torch.float32, device=dev)  # compact depths for the list builder
        self.offsets = torch.empty(V * n + 1, dtype=torch.int32, device=dev) if self.with_offsets else None
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
        self.fwd_l1_ws = torch.empty(max(L.rasterize_fwd_l1_workspace_bytes(V, self.W, self.H),
                                         L.rasterize_fwd_bwd_l1_workspace_bytes(V, self.W, self.H)),
                                     dtype=torch.uint8, device=dev)
        self.end_bit = L.sort_end_bit(V, self.T)
        self.capacity = 0
        self.allocated_for = None
        self.K = 0
        self.sorted_in_alt = False
        self.device = dev
        self.set_gauss = None  # the "compact" builder's visible sets (gs_window_gaussians)
        self.set_max = 0

    def ensure_capacity(self, K: int, slack: float = 1.25):
        if K <= self.capacity and self.capacity > 0 and self.allocated_for == self.path:
            return
        cap = max(int(K * slack) + 4096, self.capacity)
        dev = self.device
        self.vals = torch.empty(cap, dtype=torch.int32, device=dev)
        self.masks = torch.empty(cap, dtype=torch.int16, device=dev)
        self.allocated_for = self.path
        if self.path == "radix":
            self.tm_ws = torch.empty(L.tile_masks_workspace_bytes(cap), dtype=torch.uint8, device=dev)
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
            return 2 * 12 * self.capacity + 6 * self.capacity + self.sort_ws.numel()
        extra = 0
        if self.path == "compact" and self.set_gauss is not None:
            extra = (self.set_gauss.numel() + self.set_off.numel()) * 4 + self.set_ws.numel()
        return 6 * self.capacity + self.tl_ws.numel() + extra

    @property
    def binned(self) -> bool:
        """Whether the lists come from gs_tile_lists (with or without the
        compacted sets)."""
        return self.path in ("binned", "compact")

    @property
    def sorted_keys(self):
        return self.keys_alt if self.sorted_in_alt else self.keys

    @property
    def sorted_vals(self):
        return self.vals_alt if self.sorted_in_alt else self.vals

    # ---- stages ------------------------------------------------------------
    def preprocess(self, params):
        """Records, rectangles, scanned counts, the compact depths, and the
        2D-gradient records of every visible (view, Gaussian) set to zero
        (the raster passes add to them)."""
        L.gs_preprocess(params, self.n, self.sh_degree, self.cams, self.rec, self.rect,
                        self.offsets if self.with_offsets else None, self.total, self.pre_ws, depth=self.depth,
                        grad2d=self.grad2d)

    def lists_without_count(self) -> bool:
        """Whether the lists can be built before K is known on the host."""
        return self.binned and self.capacity > 0 and self.lists != "radix"

    def intersections(self, read_count: bool = True):
        """Build the per-tile lists, their ranges and sub-block masks: read K
        first, or (with read_count False and lists_without_count()) build
        them with the present capacity; the overflow flag then tells whether
        K fitted."""
        self.build_lists(read_count)
        self.tile_masks()

    def tile_masks(self):
        """The lists' sub-block masks: written by the binned builder with the
        lists; computed from the finished lists on the global-sort path."""
        if self.binned:
            return
        L.gs_tile_masks(self.rec, self.n, self.ranges, self.sorted_vals, self.capacity, self.cams, self.masks,
                        self.tm_ws)

    def build_lists(self, read_count: bool = True, sticky=None):
        """The lists and ranges alone (see ``intersections``); `sticky`, a
        device flag the binned builder sets with its overflow flag."""
        if not read_count and self.lists_without_count():
            self._bin(sticky)
            return
        self.K = int(self.total.item())
        if self.K >= 2 ** 32:
            raise L.GsError(f"{self.K} intersections exceed the 32-bit key index")
        if self.lists == "auto":
            self.path = "binned" if self.V * self.n <= self.K else "compact"
        self.ensure_capacity(self.K)
        if self.binned:
            self.sorted_in_alt = False
            self._bin(None, plan=True)
            return
        L.gs_emit_intersections(self.rec, self.rect, self.offsets, self.n, self.V, self.W, self.H,
                                self.keys, self.vals, self.capacity, self.overflow)
        self.sorted_in_alt = L.gs_sort_keys(self.keys, self.vals, self.keys_alt, self.vals_alt, self.K,
                                            self.end_bit, self.sort_ws)
        L.gs_tile_ranges(self.sorted_keys, self.K, self.V * self.T, self.ranges)

    def _bin(self, sticky, plan: bool = False):
        """gs_tile_lists over every (view, Gaussian) pair, or ("compact")
        over the sets of Gaussians each view sees; `plan` (a point where K is
        read on the host anyway): read the set sizes and size the binning
        grid for them, with slack (a larger set later is still binned whole)."""
        gauss = off = None
        if self.path == "compact":
            if self.set_gauss is None:
                dev = self.device
                self.set_gauss = torch.empty(max(1, self.V * self.n), dtype=torch.int32, device=dev)
                self.set_off = torch.empty(self.V + 1, dtype=torch.int32, device=dev)
                self.set_ws = torch.empty(L.window_gaussians_workspace_bytes(self.n, self.V), dtype=torch.uint8,
                                          device=dev)
            L.gs_window_gaussians(self.rect, self.n, self.V, self.H, 0, self.TY, self.set_gauss, self.set_off,
                                  self.set_ws)
            if plan or self.set_max == 0:
                o = self.set_off.cpu().numpy().astype("int64")
                self.set_max = min(self.n, int(1.25 * int((o[1:] - o[:-1]).max(initial=0))) + 4096)
            gauss, off = self.set_gauss, self.set_off
        L.gs_tile_lists(self.rec, self.rect, self.n, self.V, self.W, self.H, self.vals, self.capacity, self.ranges,
                        self.overflow, self.tl_ws, masks=self.masks, depth=self.depth, sticky=sticky, gauss=gauss,
                        gauss_off=off, set_max=self.set_max if gauss is not None else 0)

    def rasterize(self, bg=(0.0, 0.0, 0.0)):
        L.gs_rasterize_fwd(self.rec, self.n, self.ranges, self.sorted_vals, self.masks, self.cams, bg, self.image,
                           self.T_final, self.n_contrib)

    def loss_l1(self, target):
        scale = 1.0 / (3.0 * self.H * self.W * self.V)
        L.gs_loss_l1(self.image, target, self.image.numel(), scale, self.dL, self.loss)

    def rasterize_loss_l1(self, target, bg=(0.0, 0.0, 0.0), image: bool = False, row0: int = 0,
                          rows: Optional[int] = None, accumulate: bool = False):
        """Forward raster and L1 loss in one pass (over a window of tile rows
        when given); the image is written only when asked for."""
        scale = 1.0 / (3.0 * self.H * self.W * self.V)
        L.gs_rasterize_fwd_l1(self.rec, self.n, self.ranges, self.sorted_vals, self.masks, self.cams, bg, target, scale,
                              self.image if image else None, self.T_final, self.n_contrib, self.dL, self.loss,
                              self.fwd_l1_ws, accumulate=accumulate, row0=row0, rows=rows)

    def rasterize_fwd_bwd_l1(self, target, bg=(0.0, 0.0, 0.0), outputs: bool = False, image: bool = False,
                             row0: int = 0, rows: Optional[int] = None, accumulate: bool = False,
                             accumulate_grad2d: Optional[bool] = None):
        """Forward raster, L1 loss and backward raster in one pass (over a
        window of tile rows when given): the loss and the 2D gradients (both
        zeroed first unless `accumulate`; `accumulate_grad2d` decides for the
        2D gradients alone when given); T_final, n_contrib and dL/dimage are
        written only with `outputs`, the image only with `image`."""
        scale = 1.0 / (3.0 * self.H * self.W * self.V)
        L.gs_rasterize_fwd_bwd_l1(self.rec, self.n, self.ranges, self.sorted_vals, self.masks, self.cams, bg, target,
                                  scale, self.loss, self.grad2d, self.fwd_l1_ws,
                                  image=self.image if image else None,
                                  T_final=self.T_final if outputs else None,
                                  n_contrib=self.n_contrib if outputs else None,
                                  dL_dimage=self.dL if outputs else None,
                                  accumulate=accumulate, accumulate_grad2d=accumulate_grad2d, row0=row0, rows=rows)

    def backward(self, params, grad, bg=(0.0, 0.0, 0.0)):
        L.gs_rasterize_bwd(self.rec, self.n, self.ranges, self.sorted_vals, self.masks, self.cams, bg, self.T_final,
                           self.n_contrib, self.dL, self.grad2d)
        L.gs_preprocess_bwd(params, self.n, self.sh_degree, self.cams, self.rect, self.grad2d, grad)


def spatial_order(means) -> "numpy.ndarray":
    """A storage order of the Gaussians by the Morton (Z-order) code of their
    means, 10 bits per axis over the means' bounding box (ties by index).

    The step's result does not depend on the order in which the Gaussians are
    stored, apart from the order of equal depths in a tile's list (by index)
    and the summation order of the atomics; what depends on it is locality:
    neighbouring Gaussians share tiles, so a chunk of them fills long runs of
    a tile's list, their records share cache lines in the list gathers, and a
    wave of Gaussians tends to be seen or unseen as a whole. Apply it once,
    at set-up, to the parameters (and moments): ``params[:, perm]``; the
    inverse is ``numpy.argsort(perm)``. Host code (numpy), not part of the
    step."""
    import numpy as np

    m = np.asarray(means, dtype=np.float64)
    lo, hi = m.min(axis=1, keepdims=True), m.max(axis=1, keepdims=True)
    q = np.clip(((m - lo) / np.maximum(hi - lo, 1e-30) * 1023.0).astype(np.int64), 0, 1023)

    def spread(x):  # 10 bits to every third bit of 30
        x = (x | (x << 16)) & 0x030000FF
        x = (x | (x << 8)) & 0x0300F00F
        x = (x | (x << 4)) & 0x030C30C3
        x = (x | (x << 2)) & 0x09249249
        return x

    code = spread(q[0]) | (spread(q[1]) << 1) | (spread(q[2]) << 2)
    return np.argsort(code, kind="stable")


def render(params: torch.Tensor, sh_degree: int, cams: Sequence, bg=(0.0, 0.0, 0.0)) -> torch.Tensor:
    """Forward render of ``params`` through ``cams``; returns [V][3][H][W]."""
    b = Buffers(params.shape[1], sh_degree, cams, device=params.device)
    b.preprocess(params)
    b.intersections()
    b.rasterize(bg)
    return b.image


class TrainStep:
    """Parameters, Adam state and buffers of fwd + L1 + bwd + Adam steps.

    ``t`` counts the updates applied; with ``defer_count`` a call of ``step``
    may be redone later (see the module note), and ``flush`` settles every
    step launched so far. With ``fused_adam`` (the default) the preprocess
    backward applies Adam itself (``gs_preprocess_bwd_adam``) and ``grad`` is
    not written; otherwise ``gs_preprocess_bwd`` writes ``grad`` and
    ``gs_adam_step`` follows. ``write_image`` keeps the rendered image in
    ``buf.image`` (the step itself needs only the loss gradient). With
    ``fused_raster`` (the default) forward raster, L1 loss and backward raster
    run as one pass (``gs_rasterize_fwd_bwd_l1``), which keeps T_final,
    n_contrib and dL/dimage on chip; otherwise ``gs_rasterize_fwd_l1`` and
    ``gs_rasterize_bwd`` run one after the other and write them. With
    ``state_flags`` (the default; it takes effect when eps > 0) Adam keeps a
    byte per Gaussian that says whether its moments may be non-zero, and skips
    a Gaussian whose moments are zero and that no view sees, without reading
    it: its update would leave parameters and moments unchanged.

    The memory-capped mode (``band_rows`` tile rows per window, or
    ``list_budget`` bytes for the intersection lists and their workspace)
    builds and rasterizes the image one window of tile rows at a time, so that
    the list buffers hold one window: each window bins only the Gaussians
    whose rectangles meet it (``gs_window_gaussians``), and the loss and 2D
    gradients are summed over the windows. The windows are planned from the
    per-tile-row intersection counts, read on the host at the first step and
    after an overflow only; in between no window reads anything back (an
    overflow sets the sticky flag, which voids the step's update, and the step
    is redone with a new plan)."""

    RING = 4  # steps whose count and flag may be in flight
    LIST_SLOT_BYTES = 22  # per list slot: id 4, mask 2, and the builder's two 8-byte (depth, id) copies

    def __init__(self, params: torch.Tensor, sh_degree: int, cams: Sequence, target: torch.Tensor,
                 lr=1e-3, betas=(0.9, 0.999), eps=1e-15, bg=(0.0, 0.0, 0.0),
                 m: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None, defer_count: bool = True,
                 fused_adam: bool = True, write_image: bool = False, band_rows: Optional[int] = None,
                 fused_raster: bool = True, lists: str = "auto", state_flags: bool = True,
                 list_budget: Optional[int] = None, sparse_grad=True):
        assert params.is_cuda and params.dtype == torch.float32 and params.is_contiguous()
        self.params = params
        self.sh_degree = sh_degree
        self.buf = Buffers(params.shape[1], sh_degree, cams, device=params.device, lists=lists)
        assert params.shape[0] == self.buf.P
        self.target = target.contiguous()
        self.m = torch.zeros_like(params) if m is None else m
        self.v = torch.zeros_like(params) if v is None else v
        # per Gaussian, 0 while its moments are zero (all of them when the
        # moments start at zero): a Gaussian never seen is skipped by Adam
        fresh = m is None and v is None
        self.adam_state = (torch.zeros if fresh else torch.ones)(params.shape[1], dtype=torch.uint8,
                                                                 device=params.device)
        # with the flags, Adam skips a Gaussian with zero moments that no view
        # sees (its update is the identity when eps > 0) without reading it;
        # in a spatial storage order whole waves of such Gaussians skip
        self._use_state = state_flags and eps > 0
        # the separate backward and Adam: gradients written and read only for
        # Gaussians visible in some view (a flag per Gaussian, the gradient
        # buffer [P][n]), or "compact": only their columns, stored
        # consecutively in a buffer sized for the Gaussians seen (planned from
        # a host read of their number at the first step, and again after a
        # step whose gradients did not fit: that step sets the sticky flag and
        # is redone), or dense
        if sparse_grad not in (True, False, "compact"):
            raise ValueError("sparse_grad must be True, False or 'compact'")
        self.sparse_grad = sparse_grad if not fused_adam else False
        self.compact_grad = self.sparse_grad == "compact"
        self.grad = None if fused_adam or self.compact_grad else torch.empty_like(params)
        self.visible = (torch.zeros(params.shape[1], dtype=torch.uint8, device=params.device)
                        if self.sparse_grad is True else None)
        if self.compact_grad:
            n_g = params.shape[1]
            self.seen_list = torch.empty(max(1, n_g), dtype=torch.int32, device=params.device)
            self.seen_count = torch.zeros(1, dtype=torch.int32, device=params.device)
            self.seen_ws = torch.empty(max(1, L.seen_gaussians_workspace_bytes(n_g)), dtype=torch.uint8,
                                       device=params.device)
            self.grad_ovf = torch.zeros(1, dtype=torch.int32, device=params.device)
        self.grad_stride = 0  # columns of the compact gradient (0: plan at the next step)
        self.lr, self.betas, self.eps, self.bg = lr, betas, eps, bg
        self.t = 0
        self.defer_count = defer_count
        self.fused_adam = fused_adam
        self.fused_raster = fused_raster
        self.band_rows = band_rows
        self.list_budget = list_budget
        self.windowed = band_rows is not None or list_budget is not None
        self.windows = None  # the plan: [(row0, rows)], made at the first step and after an overflow
        self.set_max = 0  # the largest window set of the plan (with slack)
        if band_rows is not None and band_rows < 1:
            raise ValueError("band_rows must be positive")
        if self.windowed:
            b = self.buf
            b.lists, b.path = "binned", "binned"
            dev = params.device
            self.win_gauss = torch.empty(max(1, b.V * b.n), dtype=torch.int32, device=dev)
            self.win_off = torch.empty(b.V + 1, dtype=torch.int32, device=dev)
            self.win_ws = torch.empty(L.window_gaussians_workspace_bytes(b.n, b.V), dtype=torch.uint8, device=dev)
        self.write_image = write_image
        dev = params.device
        # the intersection count K and the sticky flag (an unverified step
        # overflowed) side by side, so that one asynchronous copy takes both
        # to the host after a step
        self._dev_state = torch.zeros(2, dtype=torch.int64, device=dev)
        self.buf.total = self._dev_state[0:1]
        self.sticky = self._dev_state[1:2].view(torch.int32)[0:1]
        self._host = [torch.zeros(2, dtype=torch.int64, pin_memory=True) for _ in range(self.RING)]
        self._pending = []  # (t, event, host copy of K and the flag), oldest first
        self._slot = 0
        self.redone = 0  # steps redone after an overflow

    @property
    def stage_names(self):
        """The stages that ``step(marks)`` brackets, in order."""
        tail = ["preprocess_bwd_adam"] if self.fused_adam else ["preprocess_bwd", "adam"]
        if self.windowed:
            return ["preprocess", "windows"] + tail
        if self.fused_raster:
            return ["preprocess", "intersections", "tile_masks", "raster_fwd_bwd"] + tail
        return ["preprocess", "intersections", "tile_masks", "raster_fwd_loss", "raster_bwd"] + tail

    def _plan_windows(self):
        """Windows of tile rows from the per-row intersection counts of the
        step's rectangles (a host read of the rectangles): rows of band_rows,
        or the longest runs of rows whose lists, with slack, fit the budget.
        Sizes the list buffers for the largest window."""
        import numpy as np

        b = self.buf
        r = b.rect.view(b.V, b.n, 4).cpu().numpy().view(np.uint16).astype(np.int64)
        vis = (r[..., 2] > r[..., 0]) & (r[..., 3] > r[..., 1])
        y0_all, y1_all = r[..., 1], r[..., 3]
        w, y0, y1 = (r[..., 2] - r[..., 0])[vis], r[..., 1][vis], r[..., 3][vis]
        diff = np.zeros(b.TY + 1, np.int64)
        np.add.at(diff, y0, w)
        np.add.at(diff, y1, -w)
        per_row = np.cumsum(diff)[:b.TY]  # intersections in each tile row (all views)
        slack = 1.25

        def slots(k):
            return int(k * slack) + 4096

        # the window's Gaussian set and its workspace
        set_bytes = (self.win_gauss.numel() + self.win_off.numel()) * 4 + self.win_ws.numel()

        def fixed(rows):  # the builder's workspace apart from its slots, and the set
            return L.tile_lists_workspace_bytes(b.n, b.V, b.W, 16 * rows, 0) + set_bytes

        def plan(budget):
            if self.band_rows is not None:
                return [(r0, min(self.band_rows, b.TY - r0)) for r0 in range(0, b.TY, self.band_rows)]
            out, row0 = [], 0
            while row0 < b.TY:
                rows, k = 1, int(per_row[row0])
                while row0 + rows < b.TY:
                    k2 = k + int(per_row[row0 + rows])
                    if fixed(rows + 1) + self.LIST_SLOT_BYTES * slots(k2) > budget:
                        break
                    rows, k = rows + 1, k2
                if fixed(rows) + self.LIST_SLOT_BYTES * slots(k) > budget:
                    raise L.GsError(f"tile row {row0} alone needs more than the list budget of "
                                    f"{self.list_budget} bytes")
                out.append((row0, rows))
                row0 += rows
            return out

        def peak(ws_):  # the buffers are sized for the most rows and the most intersections
            k_m = max(int(per_row[a:a + n].sum()) for a, n in ws_)
            return fixed(max(n for _, n in ws_)) + self.LIST_SLOT_BYTES * slots(k_m)

        windows = plan(self.list_budget)
        if self.band_rows is None:
            budget = self.list_budget
            for _ in range(16):  # shrink the planning budget until the sizing fits too
                over = peak(windows) - self.list_budget
                if over <= 0:
                    break
                budget -= over + 4096 * self.LIST_SLOT_BYTES
                windows = plan(budget)
        k_max = max(int(per_row[a:a + n].sum()) for a, n in windows)
        rows_max = max(n for _, n in windows)
        # the most Gaussians a view's window set holds (with slack): sizes the
        # binning grid for the sets (a larger set later is still binned whole)
        set_max = 0
        for a, n_rows in windows:
            meets = vis & (y0_all < a + n_rows) & (y1_all > a)
            set_max = max(set_max, int(meets.sum(axis=1).max(initial=0)))
        self.set_max = min(b.n, int(1.25 * set_max) + 4096)
        b.K = int(per_row.sum())
        cap = slots(k_max)
        if cap != b.capacity or b.allocated_for != b.path:  # sized for this plan, never more
            b.vals = b.masks = None
            b.vals = torch.empty(cap, dtype=torch.int32, device=b.device)
            b.masks = torch.empty(cap, dtype=torch.int16, device=b.device)
            b.capacity, b.allocated_for = cap, b.path
        ws = L.tile_lists_workspace_bytes(b.n, b.V, b.W, 16 * rows_max, b.capacity)
        if getattr(b, "tl_ws", None) is None or b.tl_ws.numel() != ws:
            b.tl_ws = None
            b.tl_ws = torch.empty(ws, dtype=torch.uint8, device=b.device)
        self.windows = windows

    def _windows(self, mark):
        """The image window by window (see the class note): each window's
        Gaussian set, lists (the overflow sets the sticky flag), forward + L1
        + backward raster; no host reads unless a new plan is needed."""
        b = self.buf
        mark(0)
        b.preprocess(self.params)  # also zeroes the visible 2D-gradient records
        mark(1)
        if self.windows is None:
            self._plan_windows()
        for i, (row0, rows) in enumerate(self.windows):
            L.gs_window_gaussians(b.rect, b.n, b.V, b.H, row0, rows, self.win_gauss, self.win_off, self.win_ws)
            L.gs_tile_lists(b.rec, b.rect, b.n, b.V, b.W, b.H, b.vals, b.capacity, b.ranges, b.overflow, b.tl_ws,
                            masks=b.masks, row0=row0, rows=rows, depth=b.depth, sticky=self.sticky,
                            gauss=self.win_gauss, gauss_off=self.win_off, set_max=self.set_max)
            # the loss is overwritten by the first window and added to by the others
            if self.fused_raster:
                b.rasterize_fwd_bwd_l1(self.target, self.bg, outputs=self.write_image, image=self.write_image,
                                       row0=row0, rows=rows, accumulate=i > 0, accumulate_grad2d=True)
                continue
            b.rasterize_loss_l1(self.target, self.bg, image=self.write_image, row0=row0, rows=rows,
                                accumulate=i > 0)
            L.gs_rasterize_bwd(b.rec, b.n, b.ranges, b.sorted_vals, b.masks, b.cams, self.bg, b.T_final, b.n_contrib,
                               b.dL, b.grad2d, accumulate=True, row0=row0, rows=rows)
        mark(2)

    def _compact_backward(self, skip, deferred, mark, m0):
        """The separate backward into the compact gradient, then Adam from it.
        A deferred step does not read the number of Gaussians seen (except to
        plan): a list longer than the buffer sets the sticky flag, and the
        step is redone. Otherwise the number is read and the buffer grown."""
        b = self.buf
        L.gs_seen_gaussians(b.rect, b.n, b.V, self.seen_list, self.seen_count, self.seen_ws)
        plan = self.grad_stride == 0
        if plan or not deferred:
            seen = int(self.seen_count.item())
            if plan or seen > self.grad_stride:
                # room for the Gaussians seen and some more (a moving view)
                self.grad_stride = max(1, min(b.n, int(1.25 * seen) + 4096))
                self.grad = None
                self.grad = torch.empty((b.P, self.grad_stride), dtype=torch.float32, device=b.device)
        L.gs_preprocess_bwd_compact(self.params, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, self.seen_list,
                                    self.seen_count, self.grad_stride, self.grad,
                                    self.sticky if deferred else self.grad_ovf)
        mark(m0)
        L.gs_adam_step_compact(self.params, self.grad, self.grad_stride, self.seen_list, self.seen_count, self.m,
                               self.v, b.n, b.P, b.rect, b.V, self.lr, self.betas[0], self.betas[1], self.eps, self.t,
                               state=self.adam_state if self._use_state else None, skip=skip)

    def list_bytes(self) -> int:
        """Bytes of the intersection lists and their workspaces (in the
        memory-capped mode also the window's Gaussian set)."""
        b = self.buf
        extra = 0
        if self.windowed:
            extra = (self.win_gauss.numel() + self.win_off.numel()) * 4 + self.win_ws.numel()
        return b.workspace_bytes() + extra

    def step(self, marks=None):
        """One step. `marks`, if given, holds len(stage_names) + 1 events,
        recorded on the stream around the stages."""
        b = self.buf
        self._settle(block=len(self._pending) >= self.RING - 1)
        mark = (lambda i: marks[i].record()) if marks is not None else (lambda i: None)
        deferred = self.defer_count and (self.windowed or b.lists_without_count())
        self.t += 1
        if self.windowed:
            self._windows(mark)
            m0 = 3
        else:
            mark(0)
            b.preprocess(self.params)  # also zeroes the visible 2D-gradient records
            mark(1)
            # an overflow of the lists also sets the sticky flag, which voids
            # this step's update and every later one until it is checked
            b.build_lists(read_count=not deferred, sticky=self.sticky if deferred else None)
            mark(2)
            b.tile_masks()
            mark(3)
            if self.fused_raster:
                # the loss is overwritten, the 2D gradients added to the
                # records the preprocess zeroed
                b.rasterize_fwd_bwd_l1(self.target, self.bg, outputs=self.write_image, image=self.write_image,
                                       accumulate=False, accumulate_grad2d=True)
                mark(4)
                m0 = 5
            else:
                b.rasterize_loss_l1(self.target, self.bg, image=self.write_image)
                mark(4)
                L.gs_rasterize_bwd(b.rec, b.n, b.ranges, b.sorted_vals, b.masks, b.cams, self.bg, b.T_final,
                                   b.n_contrib, b.dL, b.grad2d, accumulate=True)
                mark(5)
                m0 = 6
        skip = self.sticky if deferred else None
        if self.fused_adam:
            L.gs_preprocess_bwd_adam(self.params, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, self.m, self.v, self.lr,
                                     self.betas[0], self.betas[1], self.eps, self.t, skip=skip,
                                     state=self.adam_state if self._use_state else None)
        elif self.compact_grad:
            self._compact_backward(skip, deferred, mark, m0)
        else:
            L.gs_preprocess_bwd(self.params, b.n, b.sh_degree, b.cams, b.rect, b.grad2d, self.grad,
                                visible=self.visible)
            mark(m0)
            if self.sparse_grad:
                L.gs_adam_step_visible(self.params, self.grad, self.m, self.v, b.n, b.P, self.visible, self.lr,
                                       self.betas[0], self.betas[1], self.eps, self.t,
                                       state=self.adam_state if self._use_state else None, skip=skip)
            else:
                args = (self.params, self.grad, self.m, self.v, self.params.numel(), self.lr, self.betas[0],
                        self.betas[1], self.eps, self.t)
                if deferred:
                    L.gs_adam_step_unless(*args, skip)
                else:
                    L.gs_adam_step(*args)
        if deferred:
            h = self._host[self._slot]
            self._slot = (self._slot + 1) % self.RING
            h.copy_(self._dev_state, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self._pending.append((self.t, ev, h))
        mark(len(self.stage_names))

    def evaluated_pairs(self) -> int:
        """(pixel, list entry) pairs the raster passes evaluate: every entry of
        a pixel's list up to its last contributor, summed from n_contrib. The
        fused pass keeps n_contrib on chip, so one more step (an update like
        any other) writes it, window by window in the memory-capped mode --
        never a whole-image pass over a window's lists."""
        if self.fused_raster:
            keep = self.write_image
            self.write_image = True
            self.step()
            self.flush()
            self.write_image = keep
        torch.cuda.synchronize()
        return int(self.buf.n_contrib.sum(dtype=torch.int64))

    def flush(self):
        """Settle every launched step (waits for the GPU)."""
        while self._pending:
            self._settle(block=True)

    def _settle(self, block: bool):
        """Check the oldest launched steps' copied K and flag, in order."""
        b = self.buf
        while self._pending:
            t, ev, h = self._pending[0]
            if not ev.query():
                if not block:
                    return
                ev.synchronize()
                block = False  # one wait frees a slot
            self._pending.pop(0)
            b.K = int(h[0])
            if int(h[1]) != 0:  # the flag (the upper half of the word is never written)
                # step t is the first whose lists overflowed: every update from
                # it on was skipped, so redo from step t with room for K
                torch.cuda.synchronize()
                self.redone += self.t - (t - 1)
                self._pending.clear()
                self.sticky.zero_()
                if self.windowed:
                    self.windows = None  # a new plan (and list buffers) at the next step
                else:
                    b.ensure_capacity(b.K, slack=1.5)
                self.grad_stride = 0  # the compact gradient too
                self.t = t - 1
                return
