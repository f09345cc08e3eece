"""The experts of one MoE layer in MXFP8 on one GPU: buffers plus the call
sequence of the C ABI (quantise, then the scaled-MFMA grouped GEMM).

The pages credit MXFP8 for most of the feed-forward speed-up (bigchange.ai
pt-BR, "Três números, três denominadores"). Every GEMM operand is quantised
along that GEMM's contraction: token rows along d or F for the forward and
data-gradient GEMMs, token columns (blocks restarting at each expert's first
row) for the weight gradients, and each weight in the orientation its GEMM
reads. Outputs, and the SwiGLU in between, stay bf16.

The rows arrive grouped by expert (x_perm with group offsets on the device),
as in the pages' expert-parallel microbenchmark; routing, permute and combine
are the bf16 layer's and are not repeated here.
"""
from __future__ import annotations

import weakref
from typing import Dict, Sequence

import torch

from . import _lib as L


class WeightVersion:
    """Which weight tensors, at which in-place version, a set of quantised
    copies was made from. A later call matches only with the very same tensor
    objects (held by weak reference, so a freed tensor never matches, even if
    a new one reuses its memory) and no in-place write since (torch's version
    counter)."""

    def __init__(self):
        self._refs = None
        self._versions = None

    def matches(self, ws: Sequence[torch.Tensor]) -> bool:
        if self._refs is None or len(ws) != len(self._refs):
            return False
        return all(r() is w and w._version == v for r, w, v in zip(self._refs, ws, self._versions))

    def record(self, ws: Sequence[torch.Tensor]):
        self._refs = [weakref.ref(w) for w in ws]
        self._versions = [w._version for w in ws]

    def clear(self):
        self._refs = self._versions = None


class _Q:
    """Codes [rows, cols] and scales (rows * cols / 32 bytes, in the library's
    grouped layout) of one quantised operand."""

    def __init__(self, rows: int, cols: int, dev):
        self.q = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
        self.s = torch.empty(rows * cols // 32, dtype=torch.uint8, device=dev)
        self.t = L.MxTensor(self.q, self.s)


class MxExperts:
    def __init__(self, n_rows: int, d: int, E: int, F: int, device: str = "cuda", outputs: bool = True,
                 bf16_intermediates: bool = True):
        """outputs=False leaves the bf16 results (g, u, h, y_perm, dg, du,
        dx_perm, dw_*) for the caller to assign. bf16_intermediates=False
        writes H, dG and dU only as the MXFP8 copies the next GEMMs read (the
        copies, and every output and gradient, are the same bits either way;
        h, dg and du stay None)."""
        if d % 256 or F % 256:
            raise ValueError("d and F must be multiples of 256")
        self.n, self.d, self.E, self.F = n_rows, d, E, F
        dev = torch.device(device)
        bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
        n = n_rows
        self.P = L.moe_mx_col_stride(n, E)
        # forward operands
        self.xq = _Q(n, d, dev)              # x_perm rows, blocks along d
        self.wg_c = _Q(F, E * d, dev)        # W_gate columns: [F][E*d], blocks along d
        self.wu_c = _Q(F, E * d, dev)
        self.hq = _Q(n, F, dev)              # H rows
        self.wd_c = _Q(d, E * F, dev)        # W_down columns: [d][E*F], blocks along F
        # data-gradient operands
        self.dyq = _Q(n, d, dev)
        self.wd_r = _Q(E * F, d, dev)        # W_down rows, blocks along d
        self.dgq, self.duq = _Q(n, F, dev), _Q(n, F, dev)
        self.wg_r, self.wu_r = _Q(E * d, F, dev), _Q(E * d, F, dev)
        # weight-gradient operands: token columns, blocks along each expert's rows
        self.x_c = _Q(d, self.P, dev)
        self.h_c = _Q(F, self.P, dev)
        self.dy_c = _Q(d, self.P, dev)
        self.dg_c, self.du_c = _Q(F, self.P, dev), _Q(F, self.P, dev)
        # bf16 results
        self.bf16_intermediates = bf16_intermediates
        self.h = self.dg = self.du = None
        if outputs:
            self.g, self.u = bf(n, F), bf(n, F)
            self.y_perm = bf(n, d)
            if bf16_intermediates:
                self.h = bf(n, F)
                self.dg, self.du = bf(n, F), bf(n, F)
            self.dx_perm = bf(n, d)
            self.dw_gate, self.dw_up, self.dw_down = bf(E, d, F), bf(E, d, F), bf(E, F, d)
        # weight-gradient workspace (tile split and padded column starts); the
        # GEMMs run in order on one stream, so one buffer serves them all
        wgrad = L.make_mx_gg_desc(L.MOE_GG_WGRAD_GATE_UP, E, d, F, n, None, self.P)
        self.ws = torch.empty((L.moe_grouped_gemm_mx_workspace_bytes(wgrad) + 3) // 4, dtype=torch.int32,
                              device=dev)
        self.hook = None
        self._wver = WeightVersion()   # which weights the quantised copies hold

    def _mark(self, name: str):
        if self.hook is not None:
            self.hook(name)

    def _gg(self, op, **kw):
        desc = L.make_mx_gg_desc(op, self.E, self.d, self.F, self.n, self.offsets, self.P, ws=self.ws, **kw)
        L.moe_grouped_gemm_mx(desc)

    # ------------------------------------------------------------------ steps
    def quantize_weights(self, w_gate, w_up, w_down, force: bool = False) -> bool:
        """Both orientations of each weight in one pass. The weights change
        once per optimiser step, not per micro-batch: when the same tensor
        objects come back unmodified (no in-place write since, by torch's
        version counter) the quantised copies are current and nothing runs.
        A different tensor object always requantises, even at the same
        address. Writes that bypass torch's version counter need
        invalidate_weights() or force=True. Returns whether it quantised."""
        if not force and self._wver.matches((w_gate, w_up, w_down)):
            self._mark("mx_quantize_weights")
            return False
        E, d, F = self.E, self.d, self.F
        wg, wu, wd = w_gate.view(E * d, F), w_up.view(E * d, F), w_down.view(E * F, d)
        L.moe_mx_quantize_both(wg, self.wg_r.t, self.wg_c.t, None, E, E * d)
        L.moe_mx_quantize_both(wu, self.wu_r.t, self.wu_c.t, None, E, E * d)
        L.moe_mx_quantize_both(wd, self.wd_r.t, self.wd_c.t, None, E, E * F)
        self._wver.record((w_gate, w_up, w_down))
        self._mark("mx_quantize_weights")
        return True

    def invalidate_weights(self):
        """Forget which weights the quantised copies hold: the next forward
        quantises again."""
        self._wver.clear()

    def _both(self, src, rows_out, cols_out):
        L.moe_mx_quantize_both(src, rows_out.t, cols_out.t, self.offsets, self.E, self.P)

    def forward(self, x_perm, offsets, w_gate, w_up, w_down):
        self.x_perm, self.offsets = x_perm, offsets
        self.quantize_weights(w_gate, w_up, w_down)
        self._both(x_perm, self.xq, self.x_c)
        self._mark("mx_quantize_x")
        return self.forward_quantized()

    def forward_quantized(self):
        """The forward GEMMs once xq and x_c hold the quantised rows and the
        weights are quantised (the routed layer fills xq and x_c in its
        permute)."""
        # the epilogue also writes H quantised in both orientations (for the
        # down projection and its weight gradient)
        self._gg(L.MOE_GG_FWD_GATE_UP, a0=self.xq.t, b0=self.wg_c.t, b1=self.wu_c.t,
                 out0=self.g, out1=self.u, out2=self.h, qo0_rows=self.hq.t, qo0_cols=self.h_c.t)
        self._mark("mx_fwd_gate_up")
        self._gg(L.MOE_GG_FWD_DOWN, a0=self.hq.t, b0=self.wd_c.t, out0=self.y_perm)
        self._mark("mx_fwd_down")
        return self.y_perm

    def backward(self, dy_perm):
        self.backward_data(dy_perm)
        self.backward_weights()
        return self.dx_perm

    def backward_data(self, dy_perm):
        """Quantises dY (both orientations: the weight gradients read the
        token columns later) and runs the two data-gradient GEMMs; the first
        one's epilogue writes dG and dU already quantised in both orientations."""
        self._both(dy_perm, self.dyq, self.dy_c)
        self._mark("mx_quantize_dy")
        # the epilogue also writes dG and dU quantised in both orientations
        self._gg(L.MOE_GG_DGRAD_DOWN, a0=self.dyq.t, b0=self.wd_r.t, g=self.g, u=self.u,
                 out0=self.dg, out1=self.du, qo0_rows=self.dgq.t, qo0_cols=self.dg_c.t,
                 qo1_rows=self.duq.t, qo1_cols=self.du_c.t)
        self._mark("mx_dgrad_down")
        self._gg(L.MOE_GG_DGRAD_GATE_UP, a0=self.dgq.t, a1=self.duq.t, b0=self.wg_r.t, b1=self.wu_r.t,
                 out0=self.dx_perm)
        self._mark("mx_dgrad_gate_up")
        return self.dx_perm

    def backward_weights(self):
        """The weight-gradient GEMMs, from the token columns quantised by
        forward_quantized and backward_data."""
        self._gg(L.MOE_GG_WGRAD_DOWN, a0=self.h_c.t, b0=self.dy_c.t, out0=self.dw_down)
        self._mark("mx_wgrad_down")
        self._gg(L.MOE_GG_WGRAD_GATE_UP, a0=self.x_c.t, b0=self.dg_c.t, b1=self.du_c.t,
                 out0=self.dw_gate, out1=self.dw_up)
        self._mark("mx_wgrad_gate_up")

    def outputs(self) -> Dict[str, torch.Tensor]:
        return dict(G=self.g, U=self.u, H=self.h, y_perm=self.y_perm, dG=self.dg, dU=self.du,
                    dx_perm=self.dx_perm, dw_gate=self.dw_gate, dw_up=self.dw_up,
                    dw_down=self.dw_down)
