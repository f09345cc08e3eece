"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and back, the tolerance metric, and oracle evaluations on subsets of rows
(each row of the layer is independent of the others until the weight
gradients, so outputs of sampled tokens or experts can be computed one by
one on the CPU at full size)."""
from __future__ import annotations

from typing import Dict, Iterable, List

import numpy as np
import torch

import oracle.moe as om
from oracle.numerics import bf16_bits_to_f64, round_bf16, round_f32

TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 3e-2}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are all-zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def assert_close(got, ref, dtype: str, name: str):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite values"
    assert e <= TOL[dtype], f"{name}: rel err {e:.3g} > {TOL[dtype]}"
    return e


def dev(a: np.ndarray, kind: str, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; kind 'bf16' takes uint16 bit patterns."""
    if kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64 / int numpy values."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    return t.numpy()


def values(a: np.ndarray, kind: str) -> np.ndarray:
    """Float64 values of a stored input array (bf16 bits or float32)."""
    return bf16_bits_to_f64(a) if kind == "bf16" else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- sampled oracle
class Weights:
    """Expert weights held as stored arrays (bf16 bits or float32), decoded
    to float64 one expert at a time: W(name, e) has shape (1, rows, cols)."""

    def __init__(self, arrays: Dict[str, np.ndarray], kind: str):
        self.arrays, self.kind = arrays, kind

    def __call__(self, name: str, e: int) -> np.ndarray:
        return values(self.arrays[name][e:e + 1], self.kind)


def token_rows(x, W: Weights, idx: np.ndarray, tokens: Iterable[int], store):
    """Expert rows of the given tokens, computed row by row: for each (t, j)
    the G, U, H and Y rows of x[t] through expert idx[t, j]."""
    out = {}
    for t in tokens:
        for j, e in enumerate(idx[t]):
            e = int(e)
            X = x[t:t + 1]
            G, U, H = om.expert_fwd_gate_up(X, W("w_gate", e), W("w_up", e), [(0, 1)], store)
            Y = om.expert_fwd_down(H, W("w_down", e), [(0, 1)], store)
            out[(t, j)] = dict(G=G[0], U=U[0], H=H[0], Y=Y[0], e=e)
    return out


def sampled_forward_backward(x, W: Weights, idx, w, dy, tokens: List[int], store, r32=round_f32,
                             keep=None):
    """y[t], dx[t] (without a router term) and dtopk_w[t] for sampled tokens;
    ``keep[t, j]`` False marks a dropped slot (padded path)."""
    rows = token_rows(x, W, idx, tokens, store)
    k = idx.shape[1]
    y, dx, dw = {}, {}, {}
    for t in tokens:
        acc = np.zeros(x.shape[1])
        gacc = np.zeros_like(acc)
        dws = np.zeros(k)
        for j in range(k):
            if keep is not None and not keep[t, j]:
                continue
            rr = rows[(t, j)]
            e = rr["e"]
            acc += w[t, j] * rr["Y"]
            dyp = store(w[t, j] * dy[t:t + 1])
            dws[j] = np.sum(dy[t] * rr["Y"])
            dG, dU = om.expert_dgrad_down(dyp, W("w_down", e), rr["G"][None], rr["U"][None],
                                          [(0, 1)], store)
            dX = om.expert_dgrad_gate_up(dG, dU, W("w_gate", e), W("w_up", e), [(0, 1)], store)
            gacc += dX[0]
        y[t] = store(acc)
        dx[t] = store(gacc)
        dw[t] = r32(dws)
    return y, dx, dw


def expert_weight_grads(x, W: Weights, meta, w, dy, experts: List[int], k: int, store,
                        capacity: int = 0):
    """dW_gate, dW_up, dW_down of sampled experts from all of their rows."""
    d = x.shape[1]
    F = W.arrays["w_gate"].shape[2]
    out = {}
    for e in experts:
        if capacity > 0:
            blk = meta["src_slot"][e * capacity:(e + 1) * capacity]
            slots = blk[blk >= 0]
        else:
            slots = meta["src_slot"][meta["offsets"][e]:meta["offsets"][e + 1]]
        n = len(slots)
        t = slots // k
        j = slots % k
        X = x[t]
        G, U, H = om.expert_fwd_gate_up(X, W("w_gate", e), W("w_up", e), [(0, n)], store)
        dYp = store(w[t, j][:, None] * dy[t])
        dG, dU = om.expert_dgrad_down(dYp, W("w_down", e), G, U, [(0, n)], store)
        dWd = om.expert_wgrad_down(H, dYp, [(0, n)], F, d, store)[0]
        dWg, dWu = om.expert_wgrad_gate_up(X, dG, dU, [(0, n)], d, F, store)
        out[e] = dict(dw_gate=dWg[0], dw_up=dWu[0], dw_down=dWd)
    return out


def wgrad_split_reference(counts, tpe: int, bk: int, xcds: int = 8, fixed: int = 3,
                          skew: float = 1.25) -> List[int]:
    """What a weight-gradient launch writes as its tile split (host logic of
    the scheduler, not of the method): tile work = K steps of bk rows + fixed;
    split[0] = 1 when the equal-count split over the XCDs leaves one above
    skew x the mean work, split[1 + x] = first tile at or after x / xcds of
    the total work."""
    work = [(int(n) + bk - 1) // bk + fixed for n in counts]
    pre = [0]
    for w_ in work:
        pre.append(pre[-1] + w_)
    E = len(counts)
    T, total = E * tpe, tpe * pre[E]

    def before(u):
        if u >= T:
            return total
        e = u // tpe
        return tpe * pre[e] + (u % tpe) * (pre[e + 1] - pre[e])

    bal = 0
    if T >= xcds:   # one workgroup per tile
        q, r = divmod(T, xcds)
        most = 0
        for x in range(xcds):
            t0 = x * (q + 1) if x < r else r * (q + 1) + (x - r) * q
            t1 = t0 + q + (1 if x < r else 0)
            most = max(most, before(t1) - before(t0))
        bal = int(np.float32(most) > np.float32(skew) * np.float32(total) / np.float32(xcds))
    out = [bal]
    for x in range(xcds + 1):
        target = total * x // xcds
        if target <= 0:
            t = 0
        elif target >= total:
            t = T
        else:
            lo = max(e for e in range(E) if tpe * pre[e] <= target)
            w_ = pre[lo + 1] - pre[lo]
            j = -(-(target - tpe * pre[lo]) // w_)
            t = (lo + 1) * tpe if j >= tpe else lo * tpe + j
        out.append(t)
    return out

