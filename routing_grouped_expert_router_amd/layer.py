"""One MoE layer on one GPU: buffers plus the call sequence of the C ABI.

PyTorch only allocates device memory and supplies the stream; every step runs
in libmoe's kernels, in this order (no device-to-host copy anywhere: group
sizes and offsets are consumed on the device, as the pages' GPU-resident
routing requires -- deniz.in, "Yeni stack nasıl çalışıyor"):

  forward   router GEMM -> top-k gate -> offsets -> permute -> grouped GEMM
            gate/up + SwiGLU -> grouped GEMM down -> weighted combine
  backward  combine adjoint -> dgrad down + SwiGLU' -> wgrad down -> dgrad
            gate/up -> wgrad gate/up -> (router: gate adjoint, router GEMM
            adjoint) -> permute adjoint (+ router share of dx)

With ``routing='given'`` the top-k ids and gate weights are inputs (the pages'
random-routed system benchmarks) and the router steps are skipped.

With ``shared_ff > 0`` the layer also has one shared expert: a SwiGLU FFN of
hidden size shared_ff applied to every token, run as a one-group grouped GEMM
over the token rows; its output is added inside the combine and its share of
dx inside the permute adjoint, so y and dx are still written once (the pages'
production configurations pair top-four routing with one shared expert:
bigchange.ai pt-BR, "O que um engenheiro pode realmente testar").

With ``mxfp8=True`` (dropless, bf16 tensors) the six expert GEMMs run in
MXFP8 (``mx_layer.MxExperts``) and the permute quantises on dispatch: the
routed rows are gathered straight into E4M3 codes and scales, in the two
orientations the GEMMs read, and never written in bf16. Routing, combine and
their adjoints are the bf16 layer's.

With ``recompute=True`` the expert activations G, U and H are not kept from
the forward for the backward: the forward's gate/up GEMM writes H alone (G
and U never reach memory), H is scratch released after the down projection,
and the backward runs the gate/up GEMM again from x_perm into scratch G, U, H
that it releases when the weight gradients are done. This is the pages'
per-layer recompute, which trades activation memory for throughput (p1
deniz.in, "Ai2'nin raporladığı sayılar"; unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन,
और मेमोरी तकनीकें"). The recomputed values are bitwise those of the forward
(the kernels are deterministic).

Memory: routing metadata and workspaces are allocated with the layer; the
tensors the forward writes (x_perm, y_perm, y and, without recompute, G, U,
H) are allocated by the first forward and the gradient buffers by the first
backward, then reused by later steps, so that the memory a forward leaves
for its backward can be read off torch's allocator. With
``keep_intermediates=False`` the backward releases, when it returns, what
only the step needed (the forward's activations and outputs and its own
dY_perm, dG, dU, dX_perm), as each layer of a stack would; the gradients
(dx, the weight gradients, dtopk_w, dlogits) stay.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, T: int, d: int, E: int, k: int, F: int, dtype=torch.bfloat16,
                 routing: str = "learned", capacity: int = 0, backward: bool = True,
                 device: str = "cuda", recompute: bool = False, shared_ff: int = 0,
                 mxfp8: bool = False, keep_intermediates: bool = True, mx_bf16_intermediates: bool = True):
        if routing not in ("learned", "given"):
            raise ValueError(routing)
        self.T, self.d, self.E, self.k, self.F = T, d, E, k, F
        self.dtype, self.routing, self.capacity = dtype, routing, capacity
        self.recompute = recompute
        self.keep_intermediates = keep_intermediates
        self.R = T * k
        self.n_rows = E * capacity if capacity > 0 else self.R
        self.dev = dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        nr = self.n_rows
        if routing == "learned":
            self.logits = e(T, E, dt=f32)
            self.topk_idx = e(T, k, dt=i32)
            self.topk_w = e(T, k, dt=f32)
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.row_of = e(self.R, dt=i32)
        self.src_slot = e(nr, dt=i32)
        self.n_dropped = e(1, dt=i32)
        self.err_flag = torch.zeros(1, dtype=i32, device=dev)
        ws = max(L.moe_offsets_workspace_bytes(T, k, E), 16)
        self.ws_offsets = e((ws + 15) // 16 * 4, dt=i32)
        # Grouped-GEMM workspace (the weight-gradient tile split, and the partial sums of a
        # weight gradient whose K is split); one buffer, sized for the largest weight-gradient
        # launch of the routed and the shared experts, serves every launch because they all
        # run in order on one stream.
        gdt = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
        wsb = 4
        for op in (L.MOE_GG_WGRAD_DOWN, L.MOE_GG_WGRAD_GATE_UP):
            wsb = max(wsb, L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, gdt, E, d, F, nr, capacity)))
            if shared_ff > 0:
                wsb = max(wsb, L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, gdt, 1, d, shared_ff, T, 0)))
        self.ws_gg = e((wsb + 15) // 16 * 4, dt=i32)
        self.has_bwd = backward
        if backward and routing == "learned":
            wsr = max(L.moe_router_bwd_workspace_bytes(T, d, E), 16)
            self.ws_router = e((wsr + 15) // 16 * 4, dt=f32)
        # activations and gradients: allocated on first use (see the module notes)
        self.x_perm = self.g = self.u = self.h = self.y_perm = self.y = None
        self.dy_perm = self.dtopk_w = self.dg = self.du = self.dx_perm = self.dx = None
        self.dw_gate = self.dw_up = self.dw_down = self.dlogits = self.dw_r = None
        self.mxfp8 = mxfp8
        if mxfp8:
            if capacity > 0 or dtype != torch.bfloat16 or recompute or shared_ff > 0:
                raise ValueError("the MXFP8 layer is dropless bf16, without recompute or shared expert")
            from .mx_layer import MxExperts
            self.mx = MxExperts(self.n_rows, d, E, F, device=device, outputs=False,
                                bf16_intermediates=mx_bf16_intermediates)
        self.shared_ff = shared_ff
        if shared_ff > 0:
            Fs = shared_ff
            self.offsets_s = torch.tensor([0, T], dtype=i32, device=dev)
            self.g_s, self.u_s, self.h_s = e(T, Fs), e(T, Fs), e(T, Fs)
            self.y_s = e(T, d)
            if backward:
                self.dg_s, self.du_s = e(T, Fs), e(T, Fs)
                self.dx_s = e(T, d)
                self.dw_gate_s, self.dw_up_s, self.dw_down_s = e(d, Fs), e(d, Fs), e(Fs, d)
        self._dt = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
        # optional callable(stage_name) run after each stage is enqueued (used
        # by the benchmark to record per-stage events)
        self.hook = None

    def _new(self, *shape, dt=None):
        return torch.empty(*shape, dtype=self.dtype if dt is None else dt, device=self.dev)

    def forward_buffers(self):
        """Tensors the forward writes: x_perm (not for MXFP8, whose permute
        writes quantised rows only), y_perm, y and, unless recomputing, G, U, H."""
        nr, d, F = self.n_rows, self.d, self.F
        if self.y is None:
            if not self.mxfp8:
                self.x_perm = self._new(nr, d)
            self.y_perm, self.y = self._new(nr, d), self._new(self.T, d)
        if not self.recompute and self.g is None:
            self.g, self.u = self._new(nr, F), self._new(nr, F)
            if not (self.mxfp8 and not self.mx.bf16_intermediates):   # else H only as MXFP8 copies
                self.h = self._new(nr, F)
        if self.mxfp8:   # the MXFP8 expert GEMMs write into the layer's buffers
            self.mx.g, self.mx.u, self.mx.h, self.mx.y_perm = self.g, self.u, self.h, self.y_perm

    def backward_buffers(self):
        """Gradient buffers (kept across steps) and the backward's scratch."""
        nr, d, F, E, T = self.n_rows, self.d, self.F, self.E, self.T
        if self.dy_perm is None:
            self.dy_perm, self.dx_perm = self._new(nr, d), self._new(nr, d)
            if not (self.mxfp8 and not self.mx.bf16_intermediates):   # else dG, dU only as MXFP8 copies
                self.dg, self.du = self._new(nr, F), self._new(nr, F)
        if self.dx is None:
            self.dx = self._new(T, d)
            self.dtopk_w = self._new(T, self.k, dt=torch.float32)
            self.dw_gate, self.dw_up, self.dw_down = self._new(E, d, F), self._new(E, d, F), self._new(E, F, d)
            if self.routing == "learned":
                self.dlogits = self._new(T, E, dt=torch.float32)
                self.dw_r = self._new(d, E)
        if self.mxfp8:
            mx = self.mx
            mx.dg, mx.du, mx.dx_perm = self.dg, self.du, self.dx_perm
            mx.dw_gate, mx.dw_up, mx.dw_down = self.dw_gate, self.dw_up, self.dw_down

    def _mark(self, name: str):
        if self.hook is not None:
            self.hook(name)

    # ------------------------------------------------------------------ helpers
    def _gg(self, op, **tensors):
        grp = None if self.capacity > 0 else self.offsets
        desc = L.make_gg_desc(op, self._dt, self.E, self.d, self.F, self.n_rows, self.capacity,
                              grp, ws=self.ws_gg, **tensors)
        L.moe_grouped_gemm(desc)

    # ------------------------------------------------------------------ passes
    def route(self, x, w_r):
        L.moe_router_gemm(x, w_r, self.logits)
        self._mark("router_gemm")
        L.moe_route(self.logits, self.k, self.topk_idx, self.topk_w)
        self._mark("route")

    def _gg_shared(self, op, **tensors):
        desc = L.make_gg_desc(op, self._dt, 1, self.d, self.shared_ff, self.T, 0, self.offsets_s,
                              ws=self.ws_gg, **tensors)
        L.moe_grouped_gemm(desc)

    def shared_forward(self):
        self._gg_shared(L.MOE_GG_FWD_GATE_UP, x_perm=self.x, w_gate=self.w_gate_s, w_up=self.w_up_s,
                        g=self.g_s, u=self.u_s, h=self.h_s)
        self._gg_shared(L.MOE_GG_FWD_DOWN, h=self.h_s, w_down=self.w_down_s, y_perm=self.y_s)
        self._mark("gg_shared_fwd")

    def shared_backward(self, dy):
        self.shared_backward_data(dy)
        self.shared_backward_weights(dy)

    def shared_backward_data(self, dy):
        """dG_s, dU_s and the shared expert's share of dx (dx_s)."""
        self._gg_shared(L.MOE_GG_DGRAD_DOWN, dy_perm=dy, w_down=self.w_down_s, g=self.g_s, u=self.u_s,
                        dg=self.dg_s, du=self.du_s)
        self._gg_shared(L.MOE_GG_DGRAD_GATE_UP, dg=self.dg_s, du=self.du_s, w_gate=self.w_gate_s,
                        w_up=self.w_up_s, dx_perm=self.dx_s)
        self._mark("gg_shared_bwd_data")

    def shared_backward_weights(self, dy):
        self._gg_shared(L.MOE_GG_WGRAD_DOWN, h=self.h_s, dy_perm=dy, dw_down=self.dw_down_s)
        self._gg_shared(L.MOE_GG_WGRAD_GATE_UP, x_perm=self.x, dg=self.dg_s, du=self.du_s,
                        dw_gate=self.dw_gate_s, dw_up=self.dw_up_s)
        self._mark("gg_shared_bwd_weights")

    def forward(self, x, w_gate, w_up, w_down, w_r=None, topk_idx=None, topk_w=None,
                w_gate_s=None, w_up_s=None, w_down_s=None):
        self.x, self.w_gate, self.w_up, self.w_down, self.w_r = x, w_gate, w_up, w_down, w_r
        if self.shared_ff > 0:
            if w_gate_s is None or w_up_s is None or w_down_s is None:
                raise ValueError("a layer with a shared expert needs its weights")
            self.w_gate_s, self.w_up_s, self.w_down_s = w_gate_s, w_up_s, w_down_s
        self.forward_buffers()
        if self.routing == "learned":
            self.route(x, w_r)
        else:
            self.topk_idx, self.topk_w = topk_idx, topk_w
        self.metadata()
        self.permute()
        self.experts_forward()
        if self.shared_ff > 0:
            self.shared_forward()
        self.combine()
        return self.y

    def metadata(self):
        L.moe_offsets(self.topk_idx, self.E, self.capacity, self.counts, self.offsets, self.row_of,
                      self.src_slot, self.n_dropped, self.err_flag, self.ws_offsets)
        self._mark("offsets")

    def permute(self):
        if self.mxfp8:
            L.moe_permute_mx(self.x, self.k, self.src_slot, self.offsets, self.E, self.mx.P,
                             self.mx.xq.t, self.mx.x_c.t)
            self._mark("permute_mx")
            return
        L.moe_permute(self.x, self.k, self.row_of, self.src_slot if self.capacity > 0 else None,
                      self.x_perm)
        self._mark("permute")

    def experts_forward(self):
        if self.mxfp8:
            self.mx.offsets = self.offsets
            self.mx.hook = self.hook
            self.mx.quantize_weights(self.w_gate, self.w_up, self.w_down)
            self.mx.forward_quantized()
            return
        if self.recompute:
            # H alone, as scratch for the down projection; G and U are never written
            h = self._new(self.n_rows, self.F)
            self._gg(L.MOE_GG_FWD_GATE_UP, x_perm=self.x_perm, w_gate=self.w_gate, w_up=self.w_up, h=h)
            self._mark("gg_fwd_gate_up")
            self._gg(L.MOE_GG_FWD_DOWN, h=h, w_down=self.w_down, y_perm=self.y_perm)
            self._mark("gg_fwd_down")
            return
        self._gg(L.MOE_GG_FWD_GATE_UP, x_perm=self.x_perm, w_gate=self.w_gate, w_up=self.w_up,
                 g=self.g, u=self.u, h=self.h)
        self._mark("gg_fwd_gate_up")
        self._gg(L.MOE_GG_FWD_DOWN, h=self.h, w_down=self.w_down, y_perm=self.y_perm)
        self._mark("gg_fwd_down")

    def combine(self):
        L.moe_unpermute_combine(self.y_perm, self.row_of, self.topk_w, self.y,
                                y_add=self.y_s if self.shared_ff > 0 else None)
        self._mark("combine")

    def backward(self, dy):
        """Data gradients first (dx is what the layer below, or an expert-
        parallel exchange, waits on, and each data-gradient GEMM reads what
        the one before it just wrote), weight gradients last."""
        self.backward_buffers()
        # with src_slot the adjoint runs in row order (see moe_unpermute_combine_bwd)
        L.moe_unpermute_combine_bwd(dy, self.y_perm, self.topk_w, self.row_of, self.src_slot,
                                    self.dy_perm, self.dtopk_w)
        self._mark("combine_bwd")
        self.experts_backward_data()
        dx_add = None
        if self.shared_ff > 0:
            self.shared_backward_data(dy)
            dx_add = self.dx_s
        if self.routing == "learned":
            L.moe_route_bwd(self.topk_idx, self.topk_w, self.dtopk_w, self.E, self.dlogits)
            self._mark("route_bwd")
            L.moe_router_gemm_bwd(self.x, self.dlogits, self.dw_r, self.ws_router)
            self._mark("router_gemm_bwd")
            L.moe_permute_bwd(self.dx_perm, self.row_of, self.k, self.dx, self.dlogits, self.w_r,
                              dx_add=dx_add)
        else:
            L.moe_permute_bwd(self.dx_perm, self.row_of, self.k, self.dx, dx_add=dx_add)
        self._mark("permute_bwd")
        self.experts_backward_weights()
        if self.shared_ff > 0:
            self.shared_backward_weights(dy)
        if not self.keep_intermediates:
            self.release_intermediates()
        return self.dx

    def release_intermediates(self):
        """Drop the step's activations and the backward's scratch (x_perm,
        G, U, H, y_perm, y, dY_perm, dG, dU, dX_perm); the next step
        allocates them again from torch's caching allocator."""
        self.x_perm = self.g = self.u = self.h = self.y_perm = self.y = None
        self.dy_perm = self.dg = self.du = self.dx_perm = None

    def experts_backward(self):
        self.experts_backward_data()
        self.experts_backward_weights()

    def experts_backward_data(self):
        """dG, dU and dx_perm (after re-running the gate/up GEMM when the
        forward kept no G, U, H)."""
        if self.mxfp8:
            self.mx.hook = self.hook
            self.mx.backward_data(self.dy_perm)
            return
        if self.recompute:
            nr, F = self.n_rows, self.F
            self.g, self.u, self.h = self._new(nr, F), self._new(nr, F), self._new(nr, F)
            self._gg(L.MOE_GG_FWD_GATE_UP, x_perm=self.x_perm, w_gate=self.w_gate, w_up=self.w_up,
                     g=self.g, u=self.u, h=self.h)
            self._mark("gg_recompute_gate_up")
        self._gg(L.MOE_GG_DGRAD_DOWN, dy_perm=self.dy_perm, w_down=self.w_down, g=self.g, u=self.u,
                 dg=self.dg, du=self.du)
        self._mark("gg_dgrad_down")
        self._gg(L.MOE_GG_DGRAD_GATE_UP, dg=self.dg, du=self.du, w_gate=self.w_gate, w_up=self.w_up,
                 dx_perm=self.dx_perm)
        self._mark("gg_dgrad_gate_up")

    def experts_backward_weights(self):
        """dW_down, dW_gate, dW_up."""
        if self.mxfp8:
            self.mx.hook = self.hook
            self.mx.backward_weights()
            return
        self._gg(L.MOE_GG_WGRAD_DOWN, h=self.h, dy_perm=self.dy_perm, dw_down=self.dw_down)
        self._mark("gg_wgrad_down")
        self._gg(L.MOE_GG_WGRAD_GATE_UP, x_perm=self.x_perm, dg=self.dg, du=self.du,
                 dw_gate=self.dw_gate, dw_up=self.dw_up)
        self._mark("gg_wgrad_gate_up")
        if self.recompute and not self.keep_intermediates:
            self.g = self.u = self.h = None   # the recomputed scratch goes at once

    def grads(self) -> Dict[str, torch.Tensor]:
        out = dict(dx=self.dx, dw_gate=self.dw_gate, dw_up=self.dw_up, dw_down=self.dw_down,
                   dtopk_w=self.dtopk_w)
        if self.shared_ff > 0:
            out.update(dw_gate_s=self.dw_gate_s, dw_up_s=self.dw_up_s, dw_down_s=self.dw_down_s)
        if self.routing == "learned":
            out.update(dlogits=self.dlogits, dw_r=self.dw_r)
        return out
