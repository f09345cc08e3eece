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
        ("qo0_rows", moe_mx_tensor), ("qo0_cols", moe_mx_tensor),
        ("qo1_rows", moe_mx_tensor), ("qo1_cols", moe_mx_tensor),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [_i]),
    "moe_abi_version": (_i, []),
    "moe_router_gemm": (_i, [_i, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_route": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_offsets_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_offsets": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_offsets_noalloc": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
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


class _HostTensor:
    """Stands in for the address of a tensor that is not in device memory; a
    call that receives one raises before reaching the library (after every
    argument's layout has been checked)."""


_HOST = _HostTensor()


def _p(t: Optional[torch.Tensor]):
    """Device address of a tensor (None -> NULL); the tensor must be a
    contiguous device tensor, since the library reads dense row-major memory."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoEError("libmoe needs contiguous tensors")
    if not t.is_cuda:
        return _HOST
    return t.data_ptr()


def _call(name: str, *args):
    """Call entry point `name` with marshalled arguments, raising MoEError for
    host tensors or a non-zero status."""
    if any(a is _HOST for a in args):
        raise MoEError(f"{name}: libmoe needs device tensors")
    _check(getattr(lib(), name)(*args), name)


_FLOATS = (torch.bfloat16, torch.float32)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported dtype {t.dtype}")


def _req(t: Optional[torch.Tensor], name: str, dtype, shape=None, optional: bool = False,
         min_numel: int = 0):
    """Check one tensor argument before its address goes to the library:
    dtype (one torch dtype or a tuple), contiguity, shape (-1 = any extent,
    an int = element count), at least min_numel elements, and device.
    Returns the address (None for an absent optional tensor). Raises MoEError
    on any mismatch, because the library would otherwise read the memory as
    if it had the declared layout."""
    if t is None:
        if optional:
            return None
        raise MoEError(f"{name} is required")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise MoEError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
    if not t.is_contiguous():
        raise MoEError(f"{name}: must be contiguous (dense row-major)")
    if isinstance(shape, int):
        if t.numel() != shape:
            raise MoEError(f"{name}: {t.numel()} elements, expected {shape}")
    elif shape is not None:
        if t.dim() != len(shape) or any(w >= 0 and w != v for w, v in zip(shape, t.shape)):
            raise MoEError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)} (-1 = any)")
    if t.numel() < min_numel:
        raise MoEError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    return _p(t)


def _nbytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


def _stream(stream=None):
    if stream is None and not torch.cuda.is_available():
        return None   # no device: the call raises on its (host) tensors first
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _fill(desc, fields):
    """Set descriptor pointer fields once every tensor has passed its layout
    check; raise if any of them is in host memory."""
    if any(v is _HOST for _, v in fields):
        raise MoEError("libmoe needs device tensors")
    for obj, name, v in ((o, n, v) for (o, n), v in fields):
        setattr(obj, name, v)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_router_gemm(x, w_r, logits, stream=None):
    T, d = x.shape
    E = w_r.shape[1]
    _call("moe_router_gemm", _dt(x), _req(x, "x", _FLOATS, (T, d)), _req(w_r, "w_r", x.dtype, (d, E)), T, d,
                                 E, _req(logits, "logits", torch.float32, (T, E)), _stream(stream))


def moe_route(logits, k, topk_idx, topk_w, stream=None):
    T, E = logits.shape
    _call("moe_route", _req(logits, "logits", torch.float32, (T, E)), T, E, k,
                           _req(topk_idx, "topk_idx", torch.int32, (T, k)),
                           _req(topk_w, "topk_w", torch.float32, (T, k)), _stream(stream))


def moe_offsets_workspace_bytes(T, k, E) -> int:
    return lib().moe_offsets_workspace_bytes(T, k, E)


def moe_offsets(topk_idx, E, capacity, counts, offsets, row_of, src_slot, n_dropped, err_flag,
                ws, stream=None):
    T, k = topk_idx.shape
    n_rows = E * capacity if capacity > 0 else T * k
    i32 = torch.int32
    _call("moe_offsets", _req(topk_idx, "topk_idx", i32, (T, k)), T, k, E, capacity,
                             _req(counts, "counts", i32, E), _req(offsets, "offsets", i32, E + 1),
                             _req(row_of, "row_of", i32, T * k), _req(src_slot, "src_slot", i32, n_rows),
                             _req(n_dropped, "n_dropped", i32, 1), _req(err_flag, "err_flag", i32, 1),
                             _p(ws), _nbytes(ws), _stream(stream))


def moe_offsets_noalloc(topk_idx, E, capacity, counts, offsets, row_of, src_slot, n_dropped, err_flag,
                        stream=None):
    T, k = topk_idx.shape
    n_rows = E * capacity if capacity > 0 else T * k
    i32 = torch.int32
    _call("moe_offsets_noalloc", _req(topk_idx, "topk_idx", i32, (T, k)), T, k, E, capacity,
          _req(counts, "counts", i32, E), _req(offsets, "offsets", i32, E + 1),
          _req(row_of, "row_of", i32, T * k), _req(src_slot, "src_slot", i32, n_rows),
          _req(n_dropped, "n_dropped", i32, 1), _req(err_flag, "err_flag", i32, 1), _stream(stream))


def moe_permute(x, k, row_of, src_slot, x_perm, stream=None):
    T, d = x.shape
    n = x_perm.shape[0]
    i32 = torch.int32
    _call("moe_permute", _dt(x), _req(x, "x", _FLOATS, (T, d)), T, d, k, _req(row_of, "row_of", i32, T * k),
                             _req(src_slot, "src_slot", i32, n, optional=True), n,
                             _req(x_perm, "x_perm", x.dtype, (n, d)), _stream(stream))


def moe_unpermute_combine(y_perm, row_of, topk_w, y, y_add=None, stream=None):
    T, k = topk_w.shape
    d = y.shape[1]
    n = y_perm.shape[0]
    _call("moe_unpermute_combine", _dt(y), _req(y_perm, "y_perm", y.dtype, (n, d)),
                                       _req(row_of, "row_of", torch.int32, T * k),
                                       _req(topk_w, "topk_w", torch.float32, (T, k)), T, k, d, n,
                                       _req(y_add, "y_add", y.dtype, (T, d), optional=True),
                                       _req(y, "y", _FLOATS, (T, d)), _stream(stream))


def moe_unpermute_combine_bwd(dy, y_perm, topk_w, row_of, src_slot, dy_perm, dtopk_w, stream=None):
    T, k = topk_w.shape
    d = dy.shape[1]
    n = y_perm.shape[0]
    i32, f32 = torch.int32, torch.float32
    _call("moe_unpermute_combine_bwd", _dt(dy), _req(dy, "dy", _FLOATS, (T, d)),
                                           _req(y_perm, "y_perm", dy.dtype, (n, d)),
                                           _req(topk_w, "topk_w", f32, (T, k)), _req(row_of, "row_of", i32, T * k),
                                           _req(src_slot, "src_slot", i32, n, optional=True), T, k, d, n,
                                           _req(dy_perm, "dy_perm", dy.dtype, (n, d)),
                                           _req(dtopk_w, "dtopk_w", f32, (T, k)), _stream(stream))


def moe_permute_bwd(dx_perm, row_of, k, dx, dlogits=None, w_r=None, dx_add=None, stream=None):
    T, d = dx.shape
    E = 0 if w_r is None else w_r.shape[1]
    n = dx_perm.shape[0]
    _call("moe_permute_bwd", _dt(dx), _req(dx_perm, "dx_perm", dx.dtype, (n, d)),
                                 _req(row_of, "row_of", torch.int32, T * k), T, k, d, n,
                                 _req(dlogits, "dlogits", torch.float32, (T, E), optional=True),
                                 _req(w_r, "w_r", dx.dtype, (d, E), optional=True), E,
                                 _req(dx_add, "dx_add", dx.dtype, (T, d), optional=True),
                                 _req(dx, "dx", _FLOATS, (T, d)), _stream(stream))


def moe_route_bwd(topk_idx, topk_w, dtopk_w, E, dlogits, stream=None):
    T, k = topk_idx.shape
    f32 = torch.float32
    _call("moe_route_bwd", _req(topk_idx, "topk_idx", torch.int32, (T, k)), _req(topk_w, "topk_w", f32, (T, k)),
                               _req(dtopk_w, "dtopk_w", f32, (T, k)), T, E, k,
                               _req(dlogits, "dlogits", f32, (T, E)), _stream(stream))


def moe_router_bwd_workspace_bytes(T, d, E) -> int:
    return lib().moe_router_bwd_workspace_bytes(T, d, E)


def moe_router_gemm_bwd(x, dlogits, dw_r, ws, stream=None):
    T, d = x.shape
    E = dlogits.shape[1]
    _call("moe_router_gemm_bwd", _dt(x), _req(x, "x", _FLOATS, (T, d)),
                                     _req(dlogits, "dlogits", torch.float32, (T, E)), T, d, E,
                                     _req(dw_r, "dw_r", x.dtype, (d, E)), _p(ws), _nbytes(ws), _stream(stream))


# elements each grouped-GEMM tensor must hold, from (E, d, F, n_rows)
_GG_NUMEL = {
    "x_perm": lambda E, d, F, n: n * d, "y_perm": lambda E, d, F, n: n * d,
    "dy_perm": lambda E, d, F, n: n * d, "dx_perm": lambda E, d, F, n: n * d,
    "g": lambda E, d, F, n: n * F, "u": lambda E, d, F, n: n * F, "h": lambda E, d, F, n: n * F,
    "dg": lambda E, d, F, n: n * F, "du": lambda E, d, F, n: n * F,
    "w_gate": lambda E, d, F, n: E * d * F, "w_up": lambda E, d, F, n: E * d * F,
    "w_down": lambda E, d, F, n: E * F * d, "dw_gate": lambda E, d, F, n: E * d * F,
    "dw_up": lambda E, d, F, n: E * d * F, "dw_down": lambda E, d, F, n: E * F * d,
}


def make_gg_desc(op, dtype, E, d, F, n_rows, capacity=0, group_offsets=None, ws=None,
                 **tensors) -> moe_gg_desc:
    desc = moe_gg_desc()
    desc.op, desc.dtype, desc.E, desc.d, desc.F = op, dtype, E, d, F
    desc.n_rows, desc.capacity = n_rows, capacity
    fields = [((desc, "group_offsets"), _req(group_offsets, "group_offsets", torch.int32, E + 1, optional=True))]
    tdt = torch.bfloat16 if dtype == MOE_BF16 else torch.float32
    for name, t in tensors.items():
        if name not in _GG_NUMEL:
            raise MoEError(f"moe_gg_desc has no tensor {name}")
        # the call touches this many elements (a larger buffer is fine)
        fields.append(((desc, name), _req(t, name, tdt, optional=True, min_numel=_GG_NUMEL[name](E, d, F, n_rows))))
    if ws is not None:
        fields.append(((desc, "ws"), _p(ws)))
        desc.ws_bytes = _nbytes(ws)
    _fill(desc, fields)
    return desc


def moe_grouped_gemm_workspace_bytes(desc: moe_gg_desc) -> int:
    return lib().moe_grouped_gemm_workspace_bytes(C.byref(desc))


def moe_grouped_gemm(desc: moe_gg_desc, stream=None):
    _call("moe_grouped_gemm", C.byref(desc), _stream(stream))


# ----------------------------------------------------------------- MXFP8
class MxTensor:
    """E4M3 codes and E8M0 scales of one quantised operand (uint8 tensors)."""

    def __init__(self, q: torch.Tensor, s: torch.Tensor):
        self.q, self.s = q, s


def moe_mx_col_stride(rows: int, n_groups: int) -> int:
    return lib().moe_mx_col_stride(rows, n_groups)


def moe_mx_quantize(src, axis, q, s, group_offsets=None, n_groups=1, col_stride=0, stream=None):
    rows, cols = src.shape
    u8 = torch.uint8
    _call("moe_mx_quantize", _req(src, "src", torch.bfloat16, (rows, cols)), rows, cols, axis,
                                 _req(group_offsets, "group_offsets", torch.int32, n_groups + 1, optional=True),
                                 n_groups, col_stride, _req(q, "q", u8), _req(s, "s", u8), _stream(stream))


def moe_mx_quantize_both(src, rows_out: MxTensor, cols_out: MxTensor, group_offsets=None, n_groups=1,
                         col_stride=0, stream=None):
    rows, cols = src.shape
    u8 = torch.uint8
    _call("moe_mx_quantize_both", _req(src, "src", torch.bfloat16, (rows, cols)), rows, cols,
                                      _req(group_offsets, "group_offsets", torch.int32, n_groups + 1, optional=True),
                                      n_groups, col_stride, _req(rows_out.q, "q_rows", u8), _req(rows_out.s, "s_rows", u8),
                                      _req(cols_out.q, "q_cols", u8), _req(cols_out.s, "s_cols", u8),
                                      _stream(stream))


def moe_permute_mx(x, k, src_slot, group_offsets, E, col_stride, rows_out: MxTensor, cols_out: MxTensor,
                   stream=None):
    T, d = x.shape
    n_rows = src_slot.shape[0]
    u8, i32 = torch.uint8, torch.int32
    _call("moe_permute_mx", _req(x, "x", torch.bfloat16, (T, d)), T, d, k, _req(src_slot, "src_slot", i32, n_rows),
                                _req(group_offsets, "group_offsets", i32, E + 1), E, n_rows, col_stride,
                                _req(rows_out.q, "q_rows", u8), _req(rows_out.s, "s_rows", u8),
                                _req(cols_out.q, "q_cols", u8), _req(cols_out.s, "s_cols", u8),
                                _stream(stream))


def make_mx_gg_desc(op, E, d, F, n_rows, group_offsets, col_stride=0, a0=None, a1=None, b0=None,
                    b1=None, g=None, u=None, out0=None, out1=None, out2=None, ws=None, qo0_rows=None,
                    qo0_cols=None, qo1_rows=None, qo1_cols=None) -> moe_mx_gg_desc:
    desc = moe_mx_gg_desc()
    desc.op, desc.E, desc.d, desc.F, desc.n_rows, desc.col_stride = op, E, d, F, n_rows, col_stride
    fields = [((desc, "group_offsets"), _req(group_offsets, "group_offsets", torch.int32, E + 1, optional=True))]
    for name, t in (("a0", a0), ("a1", a1), ("b0", b0), ("b1", b1), ("qo0_rows", qo0_rows),
                    ("qo0_cols", qo0_cols), ("qo1_rows", qo1_rows), ("qo1_cols", qo1_cols)):
        if t is not None:
            fields.append(((getattr(desc, name), "q"), _req(t.q, f"{name}.q", torch.uint8)))
            fields.append(((getattr(desc, name), "s"), _req(t.s, f"{name}.s", torch.uint8)))
    for name, t in (("g", g), ("u", u), ("out0", out0), ("out1", out1), ("out2", out2)):
        fields.append(((desc, name), _req(t, name, torch.bfloat16, optional=True)))
    if ws is not None:
        fields.append(((desc, "ws"), _p(ws)))
        desc.ws_bytes = _nbytes(ws)
    _fill(desc, fields)
    return desc


def moe_grouped_gemm_mx_workspace_bytes(desc: moe_mx_gg_desc) -> int:
    return lib().moe_grouped_gemm_mx_workspace_bytes(C.byref(desc))


def moe_grouped_gemm_mx(desc: moe_mx_gg_desc, stream=None):
    _call("moe_grouped_gemm_mx", C.byref(desc), _stream(stream))
