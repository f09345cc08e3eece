"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, the binding covers them all, and
argument errors come back synchronously with the documented codes before
anything is launched."""
import ctypes as C
import os
import re

import pytest

from routing_grouped_expert_router_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

INVALID, UNSUPPORTED, WORKSPACE, HIP_ERR = -1, -2, -3, -4


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_layer_entry_points():
    names = declared()
    for n in ("moe_route", "moe_offsets", "moe_permute", "moe_grouped_gemm",
              "moe_unpermute_combine", "moe_unpermute_combine_bwd", "moe_permute_bwd",
              "moe_route_bwd", "moe_router_gemm", "moe_router_gemm_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(L.LIB_PATH)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert sorted(L.SIGNATURES) == declared()
    lib = L.lib()
    assert lib.moe_abi_version() == 6
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(-3) == b"workspace missing or too small"
    assert lib.moe_status_string(12345) == b"unknown status"


def test_desc_layout_matches_header():
    # int op..capacity (7), pointer group_offsets, 15 tensor pointers, ws, ws_bytes
    assert C.sizeof(L.moe_gg_desc) == 7 * 4 + 4 + 8 * 17 + 8
    # int op..col_stride (6), group_offsets, 4 (codes, scales) pairs, g, u, 3 outputs
    assert C.sizeof(L.moe_mx_tensor) == 16
    # ... then ws, ws_bytes and the four epilogue-quantised (codes, scales) pairs
    assert C.sizeof(L.moe_mx_gg_desc) == 6 * 4 + 8 + 4 * 16 + 5 * 8 + 2 * 8 + 4 * 16
    assert L.moe_mx_gg_desc.a0.offset == 32 and L.moe_mx_gg_desc.g.offset == 96


FAKE = 0x1000   # 16-byte aligned, never dereferenced: every call below fails its checks first


def test_route_argument_errors():
    lib = L.lib()
    assert lib.moe_route(FAKE, 4, 2, 3, FAKE, FAKE, None) == INVALID          # k > E
    assert lib.moe_route(FAKE, 4, 8, 0, FAKE, FAKE, None) == INVALID          # k < 1
    assert lib.moe_route(None, 4, 8, 2, FAKE, FAKE, None) == INVALID          # null logits
    assert lib.moe_route(FAKE, -1, 8, 2, FAKE, FAKE, None) == INVALID
    assert lib.moe_route(FAKE, 4, 2048, 2, FAKE, FAKE, None) == UNSUPPORTED   # E > 1024
    assert lib.moe_route(FAKE, 4, 64, 17, FAKE, FAKE, None) == UNSUPPORTED    # k > 16


def test_offsets_argument_errors():
    lib = L.lib()
    need = lib.moe_offsets_workspace_bytes(100, 4, 8)
    assert need == 8 * 4
    assert lib.moe_offsets_workspace_bytes(16384, 4, 128) == 64 * 128 * 4
    args = lambda ws, nb, cap=0, k=4: (FAKE, 100, k, 8, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    assert lib.moe_offsets(*args(None, 0)) == WORKSPACE
    assert lib.moe_offsets(*args(FAKE, need - 1)) == WORKSPACE
    assert lib.moe_offsets(*args(FAKE, need, cap=-1)) == INVALID
    assert lib.moe_offsets(*args(FAKE, need, k=9)) == INVALID


def test_row_calls_argument_errors():
    lib = L.lib()
    # d not a multiple of 8
    assert lib.moe_permute(1, FAKE, 10, 12, 2, FAKE, None, 20, FAKE, None) == INVALID
    # padded layout without src_slot
    assert lib.moe_permute(1, FAKE, 10, 16, 2, FAKE, None, 25, FAKE, None) == INVALID
    # misaligned tensor
    assert lib.moe_permute(1, FAKE + 2, 10, 16, 2, FAKE, None, 20, FAKE, None) == INVALID
    # bad dtype
    assert lib.moe_unpermute_combine(7, FAKE, FAKE, FAKE, 10, 2, 16, 20, None, FAKE, None) == INVALID
    assert lib.moe_unpermute_combine(1, FAKE, FAKE, FAKE, 10, 17, 16, 20, None, FAKE, None) == UNSUPPORTED
    assert lib.moe_unpermute_combine(1, FAKE, FAKE, FAKE, 10, 2, 16, 20, FAKE + 4, FAKE, None) == INVALID
    assert lib.moe_unpermute_combine_bwd(1, FAKE, FAKE, FAKE, FAKE, None, 10, 2, 16, 21, FAKE, FAKE, None) == INVALID
    # router share needs both dlogits and w_r
    assert lib.moe_permute_bwd(1, FAKE, FAKE, 10, 2, 16, 20, FAKE, None, 8, None, FAKE, None) == INVALID
    assert lib.moe_permute_bwd(1, FAKE, FAKE, 10, 2, 16, 20, None, None, 0, FAKE + 2, FAKE, None) == INVALID
    assert lib.moe_route_bwd(FAKE, FAKE, FAKE, 10, 4, 5, FAKE, None) == INVALID


def test_router_argument_errors():
    lib = L.lib()
    assert lib.moe_router_gemm(1, FAKE, FAKE, 10, 12, 8, FAKE, None) == INVALID
    assert lib.moe_router_gemm(1, FAKE, FAKE, 10, 16, 4096, FAKE, None) == UNSUPPORTED
    need = lib.moe_router_bwd_workspace_bytes(300, 16, 8)
    assert need == 3 * 16 * 8 * 4
    assert lib.moe_router_gemm_bwd(1, FAKE, FAKE, 300, 16, 8, FAKE, FAKE, need - 4, None) == WORKSPACE


def test_grouped_gemm_argument_errors():
    mk = lambda **kw: L.make_gg_desc(**{**dict(op=L.MOE_GG_FWD_DOWN, dtype=L.MOE_BF16, E=4, d=256,
                                               F=256, n_rows=64, capacity=16), **kw})
    lib = L.lib()
    call = lambda d: lib.moe_grouped_gemm(C.byref(d), None)
    assert call(mk()) == INVALID                         # operands missing
    d = mk()
    d.h, d.w_down, d.y_perm = FAKE, FAKE, FAKE
    d.op = 17
    assert call(d) == INVALID
    d.op = L.MOE_GG_FWD_DOWN
    d.capacity = 100                                     # E * capacity > n_rows
    assert call(d) == INVALID
    d.capacity, d.d = 16, 12                             # d % 8 != 0
    assert call(d) == INVALID
    d.d, d.E = 256, 5000
    assert call(d) == UNSUPPORTED
    d.E, d.capacity, d.group_offsets = 4, 0, None        # dropless needs offsets
    assert call(d) == INVALID
    d.h = FAKE + 4                                       # misaligned
    d.capacity = 16
    assert call(d) == INVALID
    assert lib.moe_grouped_gemm(None, None) == INVALID
    # forward gate/up: g and u are both written or both NULL (h alone)
    d = mk(op=L.MOE_GG_FWD_GATE_UP)
    d.x_perm, d.w_gate, d.w_up, d.h = FAKE, FAKE, FAKE, FAKE
    d.g = FAKE
    assert call(d) == INVALID                            # u missing
    d.g, d.u = None, FAKE
    assert call(d) == INVALID                            # g missing
    d.u, d.h = FAKE, None
    d.g = FAKE
    assert call(d) == INVALID                            # h is always written


def test_grouped_gemm_workspace():
    """Only weight gradients over device-resident groups need a workspace (their tile split, and
    the partial sums when their K is split)."""
    lib = L.lib()
    for op in (L.MOE_GG_FWD_GATE_UP, L.MOE_GG_FWD_DOWN, L.MOE_GG_DGRAD_DOWN, L.MOE_GG_DGRAD_GATE_UP):
        for cap in (0, 16):
            d = L.make_gg_desc(op, L.MOE_BF16, 4, 256, 256, 64, cap)
            assert L.moe_grouped_gemm_workspace_bytes(d) == 0
    for op in (L.MOE_GG_WGRAD_DOWN, L.MOE_GG_WGRAD_GATE_UP):
        assert L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_BF16, 4, 256, 256, 64, 16)) == 0
        need = L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_BF16, 4, 256, 256, 64, 0))
        assert need >= 4 * 10 and need % 4 == 0
    # K split: a launch of fewer than 512 tiles (128 x 256 outputs each, 128 x 128 per matrix for
    # the gate/up pair) asks for min(8, ceil(512 / tiles)) binary32 partial copies of its result
    # after 256 bytes; one of 512 tiles or more, or in binary32, asks for the tile split alone
    for op, E, d, F, tiles in ((L.MOE_GG_WGRAD_DOWN, 1, 2048, 1024, 64),
                               (L.MOE_GG_WGRAD_GATE_UP, 1, 2048, 1024, 128),
                               (L.MOE_GG_WGRAD_DOWN, 4, 2048, 1024, 256),
                               (L.MOE_GG_WGRAD_GATE_UP, 3, 512, 256, 24)):
        m, n, np_ = (F, d, d) if op == L.MOE_GG_WGRAD_DOWN else (d, F, 2 * F)
        assert tiles == E * (m // 128) * (n // (256 if op == L.MOE_GG_WGRAD_DOWN else 128))
        ks = min(8, -(-512 // tiles))
        got = L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_BF16, E, d, F, 1000, 0))
        assert got == 256 + ks * E * m * np_ * 4, (op, E, got)
        assert L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_F32, E, d, F, 1000, 0)) == 64
    for op in (L.MOE_GG_WGRAD_DOWN, L.MOE_GG_WGRAD_GATE_UP):
        assert L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_BF16, 8, 2048, 1024, 1000, 0)) == 64
        assert L.moe_grouped_gemm_workspace_bytes(L.make_gg_desc(op, L.MOE_BF16, 128, 2048, 1024, 1000, 0)) == 64
    assert lib.moe_grouped_gemm_workspace_bytes(None) == 0
    d = L.make_gg_desc(L.MOE_GG_WGRAD_DOWN, L.MOE_BF16, 4, 256, 256, 64, 0)
    d.group_offsets, d.h, d.dy_perm, d.dw_down = FAKE, FAKE, FAKE, FAKE
    call = lambda d: lib.moe_grouped_gemm(C.byref(d), None)
    assert call(d) == WORKSPACE                          # no workspace
    d.ws, d.ws_bytes = FAKE, 60
    assert call(d) == WORKSPACE                          # too small for the tile split (a workspace
                                                         # of 64 bytes up to `need` runs K unsplit)
    d.ws, d.ws_bytes = FAKE + 2, need
    assert call(d) == WORKSPACE                          # misaligned


def test_mx_quantize_argument_errors():
    lib = L.lib()
    q = lambda *a: lib.moe_mx_quantize(*a, None)
    # axis 0: cols % 32, no groups, no stride
    assert q(FAKE, 8, 48, 0, None, 1, 0, FAKE, FAKE) == INVALID
    assert q(FAKE, 8, 64, 0, FAKE, 1, 0, FAKE, FAKE) == INVALID
    assert q(FAKE, 8, 64, 0, None, 1, 128, FAKE, FAKE) == INVALID
    assert q(FAKE, 8, 64, 2, None, 1, 0, FAKE, FAKE) == INVALID
    assert q(FAKE + 2, 8, 64, 0, None, 1, 0, FAKE, FAKE) == INVALID
    assert q(FAKE, 0, 128, 0, None, 1, 0, None, None) == 0           # nothing to do
    assert q(FAKE, 8, 96, 0, None, 1, 0, FAKE, FAKE) == INVALID       # cols % 128 (scale words)
    assert q(FAKE, 8, 128, 0, None, 1, 0, FAKE, FAKE + 2) == INVALID   # scales 4-byte aligned
    # axis 1: stride bound with device offsets, equal groups
    assert lib.moe_mx_col_stride(1000, 4) == 128 * (8 + 4)
    assert q(FAKE, 1000, 64, 1, FAKE, 4, 128 * 11, FAKE, FAKE) == INVALID
    assert q(FAKE, 1000, 64, 1, FAKE, 4, 128 * 12 + 64, FAKE, FAKE) == INVALID
    assert q(FAKE, 1000, 96, 1, FAKE, 4, 128 * 12, FAKE, FAKE) == INVALID   # cols % 64
    assert q(FAKE, 1024, 64, 1, None, 4, 896, FAKE, FAKE) == INVALID         # 4 groups of 256 need 1024
    assert q(FAKE, 1000, 64, 1, None, 3, 1152, FAKE, FAKE) == INVALID        # rows % groups
    assert q(FAKE, 1000, 64, 1, FAKE, 2000, 128 * 2010, FAKE, FAKE) == UNSUPPORTED


def test_mx_gemm_argument_errors():
    lib = L.lib()
    call = lambda d: lib.moe_grouped_gemm_mx(C.byref(d), None)
    t = L.MxTensor(None, None)

    def mk(**kw):
        d = L.make_mx_gg_desc(**{**dict(op=L.MOE_GG_FWD_DOWN, E=4, d=256, F=256, n_rows=64,
                                        group_offsets=None), **kw})
        return d
    d = mk()
    assert call(d) == INVALID                            # no offsets
    d.group_offsets = FAKE
    assert call(d) == INVALID                            # operands missing
    d.a0.q, d.a0.s, d.b0.q, d.b0.s, d.out0 = FAKE, FAKE, FAKE, FAKE, FAKE
    d.a0.s = FAKE + 2                                    # scales must be 4-byte aligned
    assert call(d) == INVALID
    d.a0.s = FAKE
    d.d = 384                                            # d % 256
    assert call(d) == UNSUPPORTED
    d.d, d.op = 256, L.MOE_GG_WGRAD_DOWN
    d.col_stride = 128 * 4                               # below 128 * (ceil(64/128) + E)
    assert call(d) == INVALID
    d.col_stride = 128 * 5 + 64
    assert call(d) == INVALID
    d.op = 9
    assert call(d) == INVALID
    assert lib.moe_grouped_gemm_mx(None, None) == INVALID


def test_mx_gemm_workspace():
    """The MXFP8 weight gradients need 4 * (E + 16) bytes of workspace, the other ops none."""
    lib = L.lib()
    call = lambda d: lib.moe_grouped_gemm_mx(C.byref(d), None)
    for op in (L.MOE_GG_FWD_GATE_UP, L.MOE_GG_FWD_DOWN, L.MOE_GG_DGRAD_DOWN, L.MOE_GG_DGRAD_GATE_UP):
        assert L.moe_grouped_gemm_mx_workspace_bytes(L.make_mx_gg_desc(op, 4, 256, 256, 64, None)) == 0
    for op in (L.MOE_GG_WGRAD_DOWN, L.MOE_GG_WGRAD_GATE_UP):
        for E in (1, 4, 1024):
            assert L.moe_grouped_gemm_mx_workspace_bytes(L.make_mx_gg_desc(op, E, 256, 256, 64, None)) == 4 * (E + 16)
    assert lib.moe_grouped_gemm_mx_workspace_bytes(None) == 0
    d = L.make_mx_gg_desc(L.MOE_GG_WGRAD_DOWN, 4, 256, 256, 64, None, col_stride=128 * 5)
    d.group_offsets, d.out0 = FAKE, FAKE
    d.a0.q, d.a0.s, d.b0.q, d.b0.s = FAKE, FAKE, FAKE, FAKE
    need = 4 * (4 + 16)
    assert call(d) == WORKSPACE                          # no workspace
    d.ws, d.ws_bytes = FAKE, 60
    assert call(d) == WORKSPACE                          # too small for the tile split (a workspace
                                                         # of 64 bytes up to `need` runs K unsplit)
    d.ws, d.ws_bytes = FAKE + 2, need
    assert call(d) == WORKSPACE                          # misaligned


def test_mx_quantize_both_argument_errors():
    lib = L.lib()
    q = lambda *a: lib.moe_mx_quantize_both(*a, None)
    assert q(FAKE, 100, 64, FAKE, 2, 128 * 3, FAKE, FAKE, FAKE, FAKE) == INVALID     # cols % 128
    assert q(FAKE, 100, 128, FAKE, 2, 128 * 2, FAKE, FAKE, FAKE, FAKE) == INVALID    # stride bound
    assert q(FAKE, 100, 128, None, 3, 128 * 3, FAKE, FAKE, FAKE, FAKE) == INVALID    # rows % groups
    assert q(FAKE, 100, 128, FAKE, 2, 128 * 3, FAKE, FAKE, None, FAKE) == INVALID    # missing output
    assert q(FAKE, 100, 128, FAKE, 2, 128 * 3, FAKE, FAKE + 1, FAKE, FAKE) == INVALID
    assert q(FAKE, 0, 128, FAKE, 2, 128 * 2, None, None, None, None) == 0


def test_library_never_syncs_copies_back_or_allocates():
    """Group sizes and every other routing result stay on the device: the
    library's sources call no HIP synchronisation, blocking or host copy,
    allocation or memset, and the Python layers read no device value back."""
    import pathlib
    import re
    root = pathlib.Path(__file__).resolve().parents[1] / "routing_grouped_expert_router_amd"
    bad_c = re.compile(r"\bhip(DeviceSynchronize|StreamSynchronize|EventSynchronize|StreamQuery|"
                       r"Memcpy\w*|Malloc\w*|Free\w*|Memset\w*|HostMalloc|HostRegister)\s*\(")
    files = [f for f in sorted((root / "csrc").iterdir()) if f.suffix in (".hip", ".h", ".cpp")]
    assert len(files) >= 5
    for f in files:
        m = bad_c.search(f.read_text())
        assert m is None, (f.name, m and m.group(0))
    bad_py = re.compile(r"\.(cpu|item|tolist|numpy)\(\)|synchronize\(")
    for name in ("layer.py", "mx_layer.py", "_lib.py"):
        for i, line in enumerate((root / name).read_text().splitlines(), 1):
            code = line.split("#", 1)[0]
            assert not bad_py.search(code), (name, i, line)



def test_binding_rejects_mismatched_tensors():
    """The binding checks dtype, contiguity, shape and device of every tensor
    before its address reaches the library (which reads dense row-major memory
    of the declared element type), so a wrong tensor raises instead of being
    misread."""
    import torch
    T, E, k, d = 8, 4, 2, 16
    lg = torch.zeros(T, E)
    idx32, w = torch.zeros(T, k, dtype=torch.int32), torch.zeros(T, k)
    with pytest.raises(L.MoEError, match="topk_idx: dtype torch.int64"):
        L.moe_route(lg, k, torch.zeros(T, k, dtype=torch.int64), w)       # torch.topk's default dtype
    with pytest.raises(L.MoEError, match="logits: dtype"):
        L.moe_route(lg.double(), k, idx32, w)
    with pytest.raises(L.MoEError, match="topk_w: shape"):
        L.moe_route(lg, k, idx32, torch.zeros(T, k + 1))
    with pytest.raises(L.MoEError, match="logits: must be contiguous"):
        L.moe_route(torch.zeros(E, T).t(), k, idx32, w)                    # a transposed view
    with pytest.raises(L.MoEError, match="device tensors"):
        L.moe_route(lg, k, idx32, w)                                       # right layout, host memory
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    with pytest.raises(L.MoEError, match="x_perm: dtype torch.float32"):
        L.moe_permute(x, k, torch.zeros(T * k, dtype=torch.int32), None, torch.zeros(T * k, d))
    with pytest.raises(L.MoEError, match="row_of: 8 elements"):
        L.moe_permute(x, k, torch.zeros(T, dtype=torch.int32), None, torch.zeros(T * k, d, dtype=torch.bfloat16))
    with pytest.raises(L.MoEError, match="dy: must be contiguous"):
        L.moe_unpermute_combine_bwd(torch.zeros(d, T, dtype=torch.bfloat16).t(), torch.zeros(T * k, d, dtype=torch.bfloat16),
                                    w, idx32.view(-1), None, torch.zeros(T * k, d, dtype=torch.bfloat16), w)
    # grouped-GEMM descriptors: every tensor of the descriptor's dtype and size
    F = 32
    with pytest.raises(L.MoEError, match="w_gate: dtype torch.float32"):
        L.make_gg_desc(L.MOE_GG_FWD_GATE_UP, L.MOE_BF16, E, d, F, T * k, 0,
                       torch.zeros(E + 1, dtype=torch.int32), w_gate=torch.zeros(E, d, F))
    with pytest.raises(L.MoEError, match="g: 256 elements, at least 512 needed"):
        L.make_gg_desc(L.MOE_GG_FWD_GATE_UP, L.MOE_BF16, E, d, F, T * k, 0,
                       torch.zeros(E + 1, dtype=torch.int32), g=torch.zeros(T, F, dtype=torch.bfloat16))
    with pytest.raises(L.MoEError, match="group_offsets: dtype torch.int64"):
        L.make_gg_desc(L.MOE_GG_FWD_GATE_UP, L.MOE_BF16, E, d, F, T * k, 0, torch.zeros(E + 1, dtype=torch.int64))
    with pytest.raises(L.MoEError, match="no tensor"):
        L.make_gg_desc(L.MOE_GG_FWD_GATE_UP, L.MOE_BF16, E, d, F, T * k, 0, None, w_gat=torch.zeros(1))


def test_offsets_noalloc_argument_errors():
    """The no-allocation routing-metadata call checks its arguments like
    moe_offsets and rejects sizes whose histogram exceeds its static array,
    before touching the device."""
    lib = L.lib()
    f = lambda T, k, E, cap=0, ptr=FAKE: lib.moe_offsets_noalloc(ptr, T, k, E, cap, FAKE, FAKE, FAKE, FAKE,
                                                                 FAKE, FAKE, None)
    assert f(100, 0, 8) == INVALID                       # k < 1
    assert f(100, 9, 8) == INVALID                       # k > E
    assert f(100, 2, 8, cap=-1) == INVALID
    assert f(100, 2, 2000) == UNSUPPORTED                # E > 1024
    limit = 1 << 20                                      # MOE_OFFSETS_NOALLOC_MAX_BYTES
    fits = lambda T, k, E: L.moe_offsets_workspace_bytes(T, k, E) <= limit
    assert not fits(600000, 4, 128) and fits(500000, 4, 128)
    assert f(600000, 4, 128) == UNSUPPORTED              # histogram beyond the static array
    assert f(300000, 1, 1024) == UNSUPPORTED
    assert lib.moe_offsets_noalloc(FAKE, 10, 2, 8, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID


def test_mx_gemm_epilogue_copies_argument_errors():
    """MXFP8 copies from the epilogue: only the forward gate/up (H) and the
    data-gradient down (dG, dU) take them, all of the op's pairs or none,
    with a valid token-column stride."""
    lib = L.lib()
    call = lambda d: lib.moe_grouped_gemm_mx(C.byref(d), None)
    E, d_, F, n = 4, 256, 256, 64
    P = 128 * (1 + E)

    def mk(op):
        desc = L.make_mx_gg_desc(op, E, d_, F, n, None, P)
        desc.group_offsets = FAKE
        for name in ("a0", "a1", "b0", "b1"):
            getattr(desc, name).q, getattr(desc, name).s = FAKE, FAKE
        desc.g, desc.u, desc.out0, desc.out1, desc.out2 = FAKE, FAKE, FAKE, FAKE, FAKE
        return desc

    d = mk(L.MOE_GG_FWD_DOWN)
    d.qo0_rows.q, d.qo0_rows.s, d.qo0_cols.q, d.qo0_cols.s = FAKE, FAKE, FAKE, FAKE
    assert call(d) == INVALID                            # an op without an epilogue copy
    d = mk(L.MOE_GG_FWD_GATE_UP)
    d.qo0_rows.q, d.qo0_rows.s = FAKE, FAKE
    assert call(d) == INVALID                            # columns missing
    d.qo0_cols.q, d.qo0_cols.s = FAKE, FAKE
    d.qo1_rows.q = FAKE
    assert call(d) == INVALID                            # a second matrix the op does not have
    d = mk(L.MOE_GG_DGRAD_DOWN)
    d.qo0_rows.q, d.qo0_rows.s, d.qo0_cols.q, d.qo0_cols.s = FAKE, FAKE, FAKE, FAKE
    assert call(d) == INVALID                            # dU's copies missing
    d.qo1_rows.q, d.qo1_rows.s, d.qo1_cols.q, d.qo1_cols.s = FAKE, FAKE, FAKE, FAKE
    d.col_stride = 128 * E                               # below the stride bound
    assert call(d) == INVALID
    d.col_stride = P
    d.qo1_cols.s = FAKE + 1                              # misaligned scales
    assert call(d) == INVALID
    # with the copies given, the bf16 tensor they come from may be left out:
    # validation passes (on a host without a GPU the launch then fails with
    # MOE_ERR_HIP); without the copies it is required
    d.qo1_cols.s = FAKE
    d.out0 = d.out1 = None
    assert call(d) == HIP_ERR                            # dG and dU only as MXFP8 copies
    d.out1 = FAKE
    assert call(d) == INVALID                            # both or neither
    d = mk(L.MOE_GG_FWD_GATE_UP)
    d.out2 = None
    assert call(d) == INVALID                            # H needed without copies
    d.qo0_rows.q, d.qo0_rows.s, d.qo0_cols.q, d.qo0_cols.s = FAKE, FAKE, FAKE, FAKE
    assert call(d) == HIP_ERR                            # H only as MXFP8 copies
    d.out0 = None
    assert call(d) == INVALID                            # G and U are always written
