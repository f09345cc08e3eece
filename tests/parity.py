"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and back, the tolerance metric, and the weight-gradient tile split the
scheduler is expected to write."""
from __future__ import annotations

from typing import List

import numpy as np
import torch

from oracle.numerics import bf16_bits_to_f64

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

