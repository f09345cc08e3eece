"""Float64 statement of one MoE layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation: T tokens, d model dim, E experts, k experts per token, F expert
hidden dim, R = T*k routed slots; slot s = t*k + j is token t's j-th choice.
All arrays are float64 holding the values of the stored tensors; ``store`` is
the rounding to the layer's storage type applied wherever a tensor is written
(see ``numerics.storer``): G, U, H, Y_perm, y, dY_perm, dG, dU, dX_perm, dx
and every weight gradient. logits, gate weights, dw and dlogits are binary32.

The pages describe the layer as a sparse mixture of experts in which each
token passes through only a few experts (deniz.in, "Hedeflediği kapasite
sorunu"); routing metadata stays on the GPU and selected rows are written
straight into each expert's input buffer, after which grouped GEMMs run the
uneven per-expert shapes (deniz.in, "Yeni stack nasıl çalışıyor"; unite.ai/hi,
"पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें"). They give no formulas; each function
below states the reading it takes.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from .numerics import mx_roundtrip, round_f32, storer


def _f32(dtype: str):
    """Rounding of the binary32 tensors (logits, gate weights, dw, dlogits);
    none in the exact 'f64' mode used for algebraic checks."""
    return (lambda a: np.asarray(a, dtype=np.float64)) if dtype == "f64" else round_f32


Groups = List[Tuple[int, int]]     # per expert: (first row, number of rows)


# ----------------------------------------------------------------------------- router
def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """logits = x . W_r, kept in binary32. The learned router of the small
    configurations (bigchange.ai pt-BR, "O que um engenheiro pode realmente
    testar"): a linear map from the token to one score per expert."""
    return round_f32(x @ w_r)


def route(logits: np.ndarray, k: int, r32=round_f32) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their gate weights.

    Reading (the pages only say tokens go to a few experts): softmax over all E
    logits, keep the k largest probabilities, renormalise them to sum to one.
    The full normaliser cancels, so w_j = exp(l_j - m) / sum_i exp(l_i - m)
    over the selected logits (m = the largest). Selection compares the binary32
    logits themselves (softmax is strictly increasing); equal logits, +0 and -0
    included, go to the lower expert id; slot j holds the j-th largest.
    Returns topk_idx [T,k] int32 and topk_w [T,k] binary32 values."""
    T, E = logits.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -logits), axis=-1)      # by -logit, then id
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return idx, r32(w)


def route_bwd(topk_idx: np.ndarray, topk_w: np.ndarray, dtopk_w: np.ndarray,
              E: int, r32=round_f32) -> np.ndarray:
    """Gradient of the logits through ``route`` with the selection held fixed.

    w = softmax over the selected logits, so d l_j = w_j (dw_j - sum_i w_i dw_i)
    for selected experts and exactly 0 for the others. Binary32 result."""
    T, k = topk_idx.shape
    s = np.sum(topk_w * dtopk_w, axis=1, keepdims=True)
    dl = np.zeros((T, E))
    np.put_along_axis(dl, topk_idx.astype(np.int64), topk_w * (dtopk_w - s), axis=1)
    return r32(dl)


def router_bwd(x: np.ndarray, w_r: np.ndarray, dlogits: np.ndarray, store):
    """dW_r = x^T dlogits (stored), and the router's share of dx,
    dlogits W_r^T (unrounded: it is summed into dx before dx is stored)."""
    return store(x.T @ dlogits), dlogits @ w_r.T


# ----------------------------------------------------------------------------- metadata
def expert_offsets(topk_idx: np.ndarray, E: int, capacity: int = 0) -> Dict[str, np.ndarray]:
    """Per-expert counts and offsets, and the slot <-> row maps, as the GPU
    keeps them (deniz.in, "Yeni stack nasıl çalışıyor": group sizes stay on
    the GPU).

    Reading: rows are expert-major and, inside an expert, in slot order (the
    order a stable counting sort gives); the rank of a slot is the number of
    earlier slots routed to the same expert.
      counts[e]   slots routed to e
      offsets     exclusive prefix sum of counts, offsets[E] = R
      dropless    row_of[s] = offsets[e_s] + rank(s)
      padded      (capacity C > 0, the common-capacity alternative of the same
                  section) row_of[s] = e_s * C + rank(s) if rank(s) < C, else
                  -1 (dropped: overflow goes in slot order)
      src_slot    inverse of row_of over R (dropless) or E*C rows (padded),
                  -1 on pad rows
      n_dropped   slots with rank >= C
    """
    flat = topk_idx.reshape(-1).astype(np.int64)
    R = flat.size
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    onehot = np.zeros((R, E), dtype=np.int32)
    onehot[np.arange(R), flat] = 1
    before = np.cumsum(onehot, axis=0) - onehot          # earlier slots, same expert
    rank = before[np.arange(R), flat].astype(np.int64)
    if capacity > 0:
        keep = rank < capacity
        row_of = np.where(keep, flat * capacity + rank, -1)
        n_rows = E * capacity
        n_dropped = int(R - keep.sum())
    else:
        row_of = offsets[flat] + rank
        n_rows = R
        n_dropped = 0
    src_slot = np.full(n_rows, -1, dtype=np.int64)
    kept = row_of >= 0
    src_slot[row_of[kept]] = np.arange(R)[kept]
    return {
        "counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
        "row_of": row_of.astype(np.int32), "src_slot": src_slot.astype(np.int32),
        "n_dropped": n_dropped, "n_rows": n_rows,
    }


def groups_of(meta: Dict[str, np.ndarray], capacity: int = 0) -> Groups:
    """Row range of each expert: [offsets[e], offsets[e+1]) dropless, or the
    uniform [e*C, (e+1)*C) of the padded path."""
    E = meta["counts"].size
    if capacity > 0:
        return [(e * capacity, capacity) for e in range(E)]
    off = meta["offsets"]
    return [(int(off[e]), int(off[e + 1] - off[e])) for e in range(E)]


# ----------------------------------------------------------------------------- row movement
def permute(x: np.ndarray, src_slot: np.ndarray, k: int) -> np.ndarray:
    """x_perm[r] = x[src_slot[r] // k]; pad rows (src_slot = -1) are zero.
    Each selected token row lands directly in its expert's block of rows
    (unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें")."""
    out = np.zeros((src_slot.size, x.shape[1]))
    live = src_slot >= 0
    out[live] = x[src_slot[live] // k]
    return out


def permute_bwd(dx_perm: np.ndarray, row_of: np.ndarray, T: int, k: int, store,
                extra: Optional[np.ndarray] = None) -> np.ndarray:
    """Adjoint of ``permute``: dx[t] = sum_j dX_perm[row_of[t,j]] (dropped
    slots add nothing), plus ``extra`` (the router's share) before storing."""
    d = dx_perm.shape[1]
    acc = np.zeros((T, d)) if extra is None else np.array(extra, dtype=np.float64)
    ro = row_of.reshape(T, k)
    for j in range(k):
        live = ro[:, j] >= 0
        acc[live] += dx_perm[ro[live, j]]
    return store(acc)


def combine(y_perm: np.ndarray, row_of: np.ndarray, topk_w: np.ndarray, T: int,
            k: int, store, extra: Optional[np.ndarray] = None) -> np.ndarray:
    """Weighted unpermute: y[t] = sum_j w[t,j] Y_perm[row_of[t,j]], dropped
    slots contribute nothing, plus ``extra`` (the shared expert's output)
    before storing. Reading: the gate weight multiplies the expert output
    after the down projection."""
    d = y_perm.shape[1]
    acc = np.zeros((T, d)) if extra is None else np.array(extra, dtype=np.float64)
    ro = row_of.reshape(T, k)
    for j in range(k):
        live = ro[:, j] >= 0
        acc[live] += topk_w[live, j:j + 1] * y_perm[ro[live, j]]
    return store(acc)


def combine_bwd(dy: np.ndarray, y_perm: np.ndarray, topk_w: np.ndarray,
                row_of: np.ndarray, n_rows: int, store, r32=round_f32):
    """Adjoint of ``combine``: dY_perm[row_of[t,j]] = w[t,j] dy[t] (stored; pad
    rows zero) and dw[t,j] = <dy[t], Y_perm[row_of[t,j]]> (binary32; 0 for
    dropped slots)."""
    T, d = dy.shape
    k = topk_w.shape[1]
    ro = row_of.reshape(T, k)
    dyp = np.zeros((n_rows, d))
    dw = np.zeros((T, k))
    for j in range(k):
        live = ro[:, j] >= 0
        rows = ro[live, j]
        dyp[rows] = store(topk_w[live, j:j + 1] * dy[live])
        dw[live, j] = np.sum(dy[live] * y_perm[rows], axis=1)
    return dyp, r32(dw)


# ----------------------------------------------------------------------------- experts
def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_fwd_gate_up(x_perm, w_gate, w_up, groups: Groups, store):
    """Per expert e over its rows X_e: G = X_e W_gate[e], U = X_e W_up[e],
    H = silu(G) * U, each stored; H is formed from the stored G and U.
    Reading: SwiGLU experts without biases (the pages name no activation)."""
    n, F = x_perm.shape[0], w_gate.shape[2]
    G, U, H = np.zeros((n, F)), np.zeros((n, F)), np.zeros((n, F))
    for e, (r0, m) in enumerate(groups):
        if m == 0:
            continue
        X = x_perm[r0:r0 + m]
        G[r0:r0 + m] = store(X @ w_gate[e])
        U[r0:r0 + m] = store(X @ w_up[e])
        H[r0:r0 + m] = store(silu(G[r0:r0 + m]) * U[r0:r0 + m])
    return G, U, H


def expert_fwd_down(h, w_down, groups: Groups, store):
    """Y_perm rows of expert e = H_e W_down[e], stored."""
    n, d = h.shape[0], w_down.shape[2]
    Y = np.zeros((n, d))
    for e, (r0, m) in enumerate(groups):
        if m:
            Y[r0:r0 + m] = store(h[r0:r0 + m] @ w_down[e])
    return Y


def expert_dgrad_down(dy_perm, w_down, G, U, groups: Groups, store):
    """dH = dY_e W_down[e]^T (not stored), then the SwiGLU derivative with
    s = sigmoid(G): dG = dH * U * s * (1 + G (1 - s)), dU = dH * G * s."""
    n, F = dy_perm.shape[0], w_down.shape[1]
    dG, dU = np.zeros((n, F)), np.zeros((n, F))
    for e, (r0, m) in enumerate(groups):
        if m == 0:
            continue
        dH = dy_perm[r0:r0 + m] @ w_down[e].T
        g, u = G[r0:r0 + m], U[r0:r0 + m]
        s = 1.0 / (1.0 + np.exp(-g))
        dG[r0:r0 + m] = store(dH * u * s * (1.0 + g * (1.0 - s)))
        dU[r0:r0 + m] = store(dH * g * s)
    return dG, dU


def expert_dgrad_gate_up(dG, dU, w_gate, w_up, groups: Groups, store):
    """dX_perm rows of expert e = dG_e W_gate[e]^T + dU_e W_up[e]^T, stored."""
    n, d = dG.shape[0], w_gate.shape[1]
    dX = np.zeros((n, d))
    for e, (r0, m) in enumerate(groups):
        if m:
            dX[r0:r0 + m] = store(dG[r0:r0 + m] @ w_gate[e].T + dU[r0:r0 + m] @ w_up[e].T)
    return dX


def expert_wgrad_down(h, dy_perm, groups: Groups, F: int, d: int, store):
    """dW_down[e] = H_e^T dY_e, stored; an expert with no rows gets zeros."""
    dW = np.zeros((len(groups), F, d))
    for e, (r0, m) in enumerate(groups):
        if m:
            dW[e] = store(h[r0:r0 + m].T @ dy_perm[r0:r0 + m])
    return dW


def expert_wgrad_gate_up(x_perm, dG, dU, groups: Groups, d: int, F: int, store):
    """dW_gate[e] = X_e^T dG_e and dW_up[e] = X_e^T dU_e, stored."""
    E = len(groups)
    dWg, dWu = np.zeros((E, d, F)), np.zeros((E, d, F))
    for e, (r0, m) in enumerate(groups):
        if m:
            X = x_perm[r0:r0 + m]
            dWg[e] = store(X.T @ dG[r0:r0 + m])
            dWu[e] = store(X.T @ dU[r0:r0 + m])
    return dWg, dWu


# ----------------------------------------------------------------------------- layer
def layer_forward(p: Dict[str, np.ndarray], k: int, dtype: str, capacity: int = 0,
                  logits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Forward pass of the whole layer.

    ``p`` holds float64 values: x [T,d], w_gate, w_up [E,d,F], w_down [E,F,d],
    and either w_r [d,E] (learned router) or topk_idx/topk_w (given routing).
    ``logits`` may be passed in to route from given binary32 logits (so that
    both sides decide the same top-k from the same numbers)."""
    store, r32 = storer(dtype), _f32(dtype)
    x = p["x"]
    T = x.shape[0]
    E = p["w_gate"].shape[0]
    out: Dict[str, np.ndarray] = {}
    if "w_r" in p:
        out["logits"] = r32(x @ p["w_r"]) if logits is None else logits
        idx, w = route(out["logits"], k, r32)
    else:
        idx, w = p["topk_idx"].astype(np.int32), r32(p["topk_w"])
    out["topk_idx"], out["topk_w"] = idx, w
    meta = expert_offsets(idx, E, capacity)
    out.update(meta)
    groups = groups_of(meta, capacity)
    xp = permute(x, meta["src_slot"], k)
    G, U, H = expert_fwd_gate_up(xp, p["w_gate"], p["w_up"], groups, store)
    Y = expert_fwd_down(H, p["w_down"], groups, store)
    ys = None
    if "w_gate_s" in p:
        out.update(shared_forward(p, store))
        ys = out["y_s"]
    y = combine(Y, meta["row_of"], w, T, k, store, ys)
    out.update(x_perm=xp, G=G, U=U, H=H, y_perm=Y, y=y)
    return out


def _shared_groups(T: int) -> Groups:
    return [(0, T)]


def shared_forward(p: Dict[str, np.ndarray], store) -> Dict[str, np.ndarray]:
    """The shared expert: one SwiGLU FFN (w_gate_s, w_up_s [d,F_s], w_down_s
    [F_s,d]) applied to every token, its stored output added to the routed
    combine. The pages' production configurations use one shared expert next
    to top-four routing (bigchange.ai pt-BR, "O que um engenheiro pode
    realmente testar"; bigchange.ai id, "Apa yang benar-benar dapat dicoba
    insinyur"); its size and placement are a reading: the same SwiGLU form as
    a routed expert, added before y is stored."""
    x = p["x"]
    grp = _shared_groups(x.shape[0])
    Gs, Us, Hs = expert_fwd_gate_up(x, p["w_gate_s"][None], p["w_up_s"][None], grp, store)
    Ys = expert_fwd_down(Hs, p["w_down_s"][None], grp, store)
    return dict(G_s=Gs, U_s=Us, H_s=Hs, y_s=Ys)


def shared_backward(p: Dict[str, np.ndarray], fwd: Dict[str, np.ndarray], dy: np.ndarray,
                    store) -> Dict[str, np.ndarray]:
    """Chain rule of ``shared_forward``: its output gradient is dy itself."""
    x = p["x"]
    d, F = p["w_gate_s"].shape
    grp = _shared_groups(x.shape[0])
    dGs, dUs = expert_dgrad_down(dy, p["w_down_s"][None], fwd["G_s"], fwd["U_s"], grp, store)
    dWds = expert_wgrad_down(fwd["H_s"], dy, grp, F, d, store)[0]
    dXs = expert_dgrad_gate_up(dGs, dUs, p["w_gate_s"][None], p["w_up_s"][None], grp, store)
    dWgs, dWus = expert_wgrad_gate_up(x, dGs, dUs, grp, d, F, store)
    return dict(dG_s=dGs, dU_s=dUs, dx_s=dXs, dw_gate_s=dWgs[0], dw_up_s=dWus[0], dw_down_s=dWds)


def layer_backward(p: Dict[str, np.ndarray], fwd: Dict[str, np.ndarray], dy: np.ndarray,
                   k: int, dtype: str, capacity: int = 0) -> Dict[str, np.ndarray]:
    """Backward pass: the chain rule of ``layer_forward`` through combine, the
    down projection, SwiGLU, the gate/up projection, the permutation and (for
    a learned router) the softmax/top-k gate and the router GEMM."""
    store, r32 = storer(dtype), _f32(dtype)
    T, d = dy.shape
    E, _, F = p["w_gate"].shape
    groups = groups_of(fwd, capacity)
    dyp, dw = combine_bwd(dy, fwd["y_perm"], fwd["topk_w"], fwd["row_of"], fwd["n_rows"],
                          store, r32)
    dG, dU = expert_dgrad_down(dyp, p["w_down"], fwd["G"], fwd["U"], groups, store)
    dWd = expert_wgrad_down(fwd["H"], dyp, groups, F, d, store)
    dXp = expert_dgrad_gate_up(dG, dU, p["w_gate"], p["w_up"], groups, store)
    dWg, dWu = expert_wgrad_gate_up(fwd["x_perm"], dG, dU, groups, d, F, store)
    out = dict(dy_perm=dyp, dtopk_w=dw, dG=dG, dU=dU, dx_perm=dXp,
               dw_gate=dWg, dw_up=dWu, dw_down=dWd)
    extra = None
    if "w_r" in p:
        dl = route_bwd(fwd["topk_idx"], fwd["topk_w"], dw, E, r32)
        dWr, extra = router_bwd(p["x"], p["w_r"], dl, store)
        out.update(dlogits=dl, dw_r=dWr)
    if "w_gate_s" in p:
        out.update(shared_backward(p, fwd, dy, store))
        extra = out["dx_s"] if extra is None else extra + out["dx_s"]
    out["dx"] = permute_bwd(dXp, fwd["row_of"], T, k, store, extra)
    return out


# ----------------------------------------------------------------------------- MXFP8 experts
def _mx_rows(a):
    """Operand values after MX quantisation along its rows' last axis."""
    return mx_roundtrip(a)


def mx_expert(X, dY, w_gate, w_up, w_down) -> Dict[str, np.ndarray]:
    """Forward and backward of one expert on its rows X [n,d] (output
    gradient rows dY [n,d]) with every GEMM operand MXFP8-quantised along
    that GEMM's contraction axis, bf16 outputs.

    The pages credit MXFP8 mostly to the feed-forward GEMMs and to moving data
    between experts (unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें").
    Reading: blocks of 32 run along K of each GEMM:
      fwd gate/up  K = d : X rows, W_gate/W_up along d
      fwd down     K = F : H rows, W_down along F
      dgrad down   K = d : dY rows, W_down along d
      dgrad g/u    K = F : dG, dU rows, W_gate/W_up along F
      wgrad        K = the expert's rows: X, H, dY, dG, dU along tokens, blocks
                   starting at the expert's first row, the last one zero-padded
    SwiGLU, its derivative and the rounding points are those of the bf16 layer."""
    st = storer("bf16")
    Xq = _mx_rows(X)
    G = st(Xq @ _mx_rows(w_gate.T).T)
    U = st(Xq @ _mx_rows(w_up.T).T)
    H = st(silu(G) * U)
    Y = st(_mx_rows(H) @ _mx_rows(w_down.T).T)
    dH = _mx_rows(dY) @ _mx_rows(w_down).T
    s = 1.0 / (1.0 + np.exp(-G))
    dG = st(dH * U * s * (1.0 + G * (1.0 - s)))
    dU = st(dH * G * s)
    dX = st(_mx_rows(dG) @ _mx_rows(w_gate).T + _mx_rows(dU) @ _mx_rows(w_up).T)
    dWd = st(_mx_rows(H.T) @ _mx_rows(dY.T).T)
    Xt = _mx_rows(X.T)
    dWg = st(Xt @ _mx_rows(dG.T).T)
    dWu = st(Xt @ _mx_rows(dU.T).T)
    return dict(G=G, U=U, H=H, y_perm=Y, dG=dG, dU=dU, dx_perm=dX, dw_gate=dWg, dw_up=dWu, dw_down=dWd)


def mx_expert_layer(x_perm, dy_perm, counts, w_gate, w_up, w_down, map_fn=map) -> Dict[str, np.ndarray]:
    """``mx_expert`` for every expert on its block of the pre-grouped rows
    (experts are independent; ``map_fn`` evaluates them, e.g. a thread
    pool's map). Experts with no rows keep zero weight gradients."""
    E, d, F = w_gate.shape
    n = x_perm.shape[0]
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    G, U, H = np.zeros((n, F)), np.zeros((n, F)), np.zeros((n, F))
    Y, dG, dU, dX = np.zeros((n, d)), np.zeros((n, F)), np.zeros((n, F)), np.zeros((n, d))
    dWg, dWu, dWd = np.zeros((E, d, F)), np.zeros((E, d, F)), np.zeros((E, F, d))
    live = [e for e in range(E) if off[e + 1] > off[e]]
    run = lambda e: mx_expert(x_perm[off[e]:off[e + 1]], dy_perm[off[e]:off[e + 1]], w_gate[e], w_up[e],
                              w_down[e])
    for e, r in zip(live, map_fn(run, live)):
        r0, r1 = int(off[e]), int(off[e + 1])
        for name, a in (("G", G), ("U", U), ("H", H), ("y_perm", Y), ("dG", dG), ("dU", dU), ("dx_perm", dX)):
            a[r0:r1] = r[name]
        dWg[e], dWu[e], dWd[e] = r["dw_gate"], r["dw_up"], r["dw_down"]
    return dict(G=G, U=U, H=H, y_perm=Y, dG=dG, dU=dU, dx_perm=dX,
                dw_gate=dWg, dw_up=dWu, dw_down=dWd)


# ----------------------------------------------------------------------------- MXFP8 routed layer
def mx_layer(p: Dict[str, np.ndarray], k: int, dy: np.ndarray,
             logits: Optional[np.ndarray] = None, map_fn=map) -> Dict[str, np.ndarray]:
    """Forward and backward of the whole routed layer with every expert GEMM
    in MXFP8 (``mx_expert_layer`` on the permuted rows) and everything else as
    in the bf16 layer: routing, offsets, permute, combine and their adjoints,
    bf16 storage. Dropless. The pages report MXFP8 against BF16 on the
    feed-forward of a routed model (bigchange.ai pt-BR, "Três números, três
    denominadores"); the routed rows are what the expert layer receives."""
    st, r32 = storer("bf16"), _f32("bf16")
    x = p["x"]
    T = x.shape[0]
    E = p["w_gate"].shape[0]
    out: Dict[str, np.ndarray] = {}
    if "w_r" in p:
        out["logits"] = r32(x @ p["w_r"]) if logits is None else logits
        idx, w = route(out["logits"], k, r32)
    else:
        idx, w = p["topk_idx"].astype(np.int32), r32(p["topk_w"])
    out["topk_idx"], out["topk_w"] = idx, w
    meta = expert_offsets(idx, E)
    out.update(meta)
    xp = permute(x, meta["src_slot"], k)
    # dY_perm rows are w * dy of their token: they do not depend on the forward
    dyp = np.zeros((meta["n_rows"], x.shape[1]))
    ro = meta["row_of"].reshape(T, k)
    for j in range(k):
        dyp[ro[:, j]] = st(w[:, j:j + 1] * dy)
    ex = mx_expert_layer(xp, dyp, meta["counts"], p["w_gate"], p["w_up"], p["w_down"], map_fn)
    out.update(x_perm=xp, dy_perm=dyp, **ex)
    out["y"] = combine(ex["y_perm"], meta["row_of"], w, T, k, st)
    _, out["dtopk_w"] = combine_bwd(dy, ex["y_perm"], w, meta["row_of"], meta["n_rows"], st, r32)
    extra = None
    if "w_r" in p:
        dl = route_bwd(idx, w, out["dtopk_w"], E, r32)
        out["dw_r"], extra = router_bwd(x, p["w_r"], dl, st)
        out["dlogits"] = dl
    out["dx"] = permute_bwd(ex["dx_perm"], meta["row_of"], T, k, st, extra)
    return out
