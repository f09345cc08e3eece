"""ctypes binding of libmoe.so: one Python function per C entry point, same
names, argument marshalling only (torch tensors -> device pointers, the
current HIP stream). Every step of the layer runs in the library's kernels.

The library must have been built (``python -m
routing_grouped_expert_router_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
(MOE_GG_FWD_GATE_UP, MOE_GG_FWD_DOWN, MOE_GG_DGRAD_DOWN, MOE_GG_DGRAD_GATE_UP,
 MOE_GG_WGRAD_DOWN, MOE_GG_WGRAD_GATE_UP) = range(6)

_vp, _i, _sz = C.c_void_p, C.c_int, C.c_size_t


class moe_gg_desc(C.Structure):
    _fields_ = [
        ("op", _i), ("dtype", _i), ("E", _i), ("d", _i), ("F", _i), ("n_rows", _i),
        ("capacity", _i), ("group_offsets", _vp),
        ("x_perm", _vp), ("g", _vp), ("u", _vp), ("h", _vp), ("y_perm", _vp),
        ("dy_perm", _vp), ("dg", _vp), ("du", _vp), ("dx_perm", _vp),
        ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp),
        ("dw_gate", _vp), ("dw_up", _vp), ("dw_down", _vp),
        ("ws", _vp), ("ws_bytes", _sz),
    ]


class moe_mx_tensor(C.Structure):
    _fields_ = [("q", _vp), ("s", _vp)]


class moe_mx_gg_desc(C.Structure):
    _fields_ = [
        ("op", _i), ("E", _i), ("d", _i), ("F", _i), ("n_rows", _i), ("col_stride", _i),
        ("group_offsets", _vp),
        ("a0", moe_mx_tensor), ("a1", moe_mx_tensor), ("b0", moe_mx_tensor), ("b1", moe_mx_tensor),
        ("g", _vp), ("u", _vp), ("out0", _vp), ("out1", _vp), ("out2", _vp),
        ("ws", _vp), ("ws_bytes", _sz),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [_i]),
    "moe_abi_version": (_i, []),
    "moe_router_gemm": (_i, [_i, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_route": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_offsets_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_offsets": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute": (_i, [_i, _vp, _i, _i, _i, _vp, _vp, _i, _vp, _vp]),
    "moe_unpermute_combine": (_i, [_i, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "moe_unpermute_combine_bwd": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "moe_permute_bwd": (_i, [_i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _vp]),
    "moe_route_bwd": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_router_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_router_gemm_bwd": (_i, [_i, _vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_workspace_bytes": (_sz, [C.POINTER(moe_gg_desc)]),
    "moe_grouped_gemm": (_i, [C.POINTER(moe_gg_desc), _vp]),
    "moe_mx_col_stride": (_i, [_i, _i]),
    "moe_mx_quantize": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp]),
    "moe_mx_quantize_both": (_i, [_vp, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_permute_mx": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm_mx_workspace_bytes": (_sz, [C.POINTER(moe_mx_gg_desc)]),
    "moe_grouped_gemm_mx": (_i, [C.POINTER(moe_mx_gg_desc), _vp]),
}

_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m routing_grouped_expert_router_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class MoEError(RuntimeError):
    pass


def _check(status: int, name: str):
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoEError(f"{name} failed: {msg} ({status})")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoEError("libmoe needs device tensors")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_router_gemm(x, w_r, logits, stream=None):
    T, d = x.shape
    E = w_r.shape[1]
    _check(lib().moe_router_gemm(_dt(x), _p(x), _p(w_r), T, d, E, _p(logits), _stream(stream)),
           "moe_router_gemm")


def moe_route(logits, k, topk_idx, topk_w, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_p(logits), T, E, k, _p(topk_idx), _p(topk_w), _stream(stream)),
           "moe_route")


def moe_offsets_workspace_bytes(T, k, E) -> int:
    return lib().moe_offsets_workspace_bytes(T, k, E)


def moe_offsets(topk_idx, E, capacity, counts, offsets, row_of, src_slot, n_dropped, err_flag,
                ws, stream=None):
    T, k = topk_idx.shape
    _check(lib().moe_offsets(_p(topk_idx), T, k, E, capacity, _p(counts), _p(offsets), _p(row_of),
                             _p(src_slot), _p(n_dropped), _p(err_flag), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_offsets")


def moe_permute(x, k, row_of, src_slot, x_perm, stream=None):
    T, d = x.shape
    _check(lib().moe_permute(_dt(x), _p(x), T, d, k, _p(row_of), _p(src_slot), x_perm.shape[0],
                             _p(x_perm), _stream(stream)), "moe_permute")


def moe_unpermute_combine(y_perm, row_of, topk_w, y, y_add=None, stream=None):
    T, k = topk_w.shape
    _check(lib().moe_unpermute_combine(_dt(y), _p(y_perm), _p(row_of), _p(topk_w), T, k, y.shape[1],
                                       y_perm.shape[0], _p(y_add), _p(y), _stream(stream)),
           "moe_unpermute_combine")


def moe_unpermute_combine_bwd(dy, y_perm, topk_w, row_of, src_slot, dy_perm, dtopk_w, stream=None):
    T, k = topk_w.shape
    _check(lib().moe_unpermute_combine_bwd(_dt(dy), _p(dy), _p(y_perm), _p(topk_w), _p(row_of),
                                           _p(src_slot), T, k, dy.shape[1], y_perm.shape[0],
                                           _p(dy_perm), _p(dtopk_w), _stream(stream)),
           "moe_unpermute_combine_bwd")


def moe_permute_bwd(dx_perm, row_of, k, dx, dlogits=None, w_r=None, dx_add=None, stream=None):
    T, d = dx.shape
    E = 0 if w_r is None else w_r.shape[1]
    _check(lib().moe_permute_bwd(_dt(dx), _p(dx_perm), _p(row_of), T, k, d, dx_perm.shape[0],
                                 _p(dlogits), _p(w_r), E, _p(dx_add), _p(dx), _stream(stream)),
           "moe_permute_bwd")


def moe_route_bwd(topk_idx, topk_w, dtopk_w, E, dlogits, stream=None):
    T, k = topk_idx.shape
    _check(lib().moe_route_bwd(_p(topk_idx), _p(topk_w), _p(dtopk_w), T, E, k, _p(dlogits),
                               _stream(stream)), "moe_route_bwd")


def moe_router_bwd_workspace_bytes(T, d, E) -> int:
    return lib().moe_router_bwd_workspace_bytes(T, d, E)


def moe_router_gemm_bwd(x, dlogits, dw_r, ws, stream=None):
    T, d = x.shape
    E = dlogits.shape[1]
    _check(lib().moe_router_gemm_bwd(_dt(x), _p(x), _p(dlogits), T, d, E, _p(dw_r), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "moe_router_gemm_bwd")


def make_gg_desc(op, dtype, E, d, F, n_rows, capacity=0, group_offsets=None, ws=None,
                 **tensors) -> moe_gg_desc:
    desc = moe_gg_desc()
    desc.op, desc.dtype, desc.E, desc.d, desc.F = op, dtype, E, d, F
    desc.n_rows, desc.capacity = n_rows, capacity
    desc.group_offsets = _p(group_offsets)
    for name, t in tensors.items():
        setattr(desc, name, _p(t))
    if ws is not None:
        desc.ws, desc.ws_bytes = _p(ws), ws.numel() * ws.element_size()
    return desc


def moe_grouped_gemm_workspace_bytes(desc: moe_gg_desc) -> int:
    return lib().moe_grouped_gemm_workspace_bytes(C.byref(desc))


def moe_grouped_gemm(desc: moe_gg_desc, stream=None):
    _check(lib().moe_grouped_gemm(C.byref(desc), _stream(stream)), "moe_grouped_gemm")


# ----------------------------------------------------------------- MXFP8
class MxTensor:
    """E4M3 codes and E8M0 scales of one quantised operand (uint8 tensors)."""

    def __init__(self, q: torch.Tensor, s: torch.Tensor):
        self.q, self.s = q, s


def moe_mx_col_stride(rows: int, n_groups: int) -> int:
    return lib().moe_mx_col_stride(rows, n_groups)


def moe_mx_quantize(src, axis, q, s, group_offsets=None, n_groups=1, col_stride=0, stream=None):
    rows, cols = src.shape
    _check(lib().moe_mx_quantize(_p(src), rows, cols, axis, _p(group_offsets), n_groups, col_stride,
                                 _p(q), _p(s), _stream(stream)), "moe_mx_quantize")


def moe_mx_quantize_both(src, rows_out: MxTensor, cols_out: MxTensor, group_offsets=None, n_groups=1,
                         col_stride=0, stream=None):
    rows, cols = src.shape
    _check(lib().moe_mx_quantize_both(_p(src), rows, cols, _p(group_offsets), n_groups, col_stride,
                                      _p(rows_out.q), _p(rows_out.s), _p(cols_out.q), _p(cols_out.s),
                                      _stream(stream)), "moe_mx_quantize_both")


def moe_permute_mx(x, k, src_slot, group_offsets, E, col_stride, rows_out: MxTensor, cols_out: MxTensor,
                   stream=None):
    T, d = x.shape
    n_rows = src_slot.shape[0]
    _check(lib().moe_permute_mx(_p(x), T, d, k, _p(src_slot), _p(group_offsets), E, n_rows, col_stride,
                                _p(rows_out.q), _p(rows_out.s), _p(cols_out.q), _p(cols_out.s),
                                _stream(stream)), "moe_permute_mx")


def make_mx_gg_desc(op, E, d, F, n_rows, group_offsets, col_stride=0, a0=None, a1=None, b0=None,
                    b1=None, g=None, u=None, out0=None, out1=None, out2=None, ws=None) -> moe_mx_gg_desc:
    desc = moe_mx_gg_desc()
    desc.op, desc.E, desc.d, desc.F, desc.n_rows, desc.col_stride = op, E, d, F, n_rows, col_stride
    desc.group_offsets = _p(group_offsets)
    for name, t in (("a0", a0), ("a1", a1), ("b0", b0), ("b1", b1)):
        if t is not None:
            getattr(desc, name).q, getattr(desc, name).s = _p(t.q), _p(t.s)
    for name, t in (("g", g), ("u", u), ("out0", out0), ("out1", out1), ("out2", out2)):
        setattr(desc, name, _p(t))
    if ws is not None:
        desc.ws, desc.ws_bytes = _p(ws), ws.numel() * ws.element_size()
    return desc


def moe_grouped_gemm_mx_workspace_bytes(desc: moe_mx_gg_desc) -> int:
    return lib().moe_grouped_gemm_mx_workspace_bytes(C.byref(desc))


def moe_grouped_gemm_mx(desc: moe_mx_gg_desc, stream=None):
    _check(lib().moe_grouped_gemm_mx(C.byref(desc), _stream(stream)), "moe_grouped_gemm_mx")
