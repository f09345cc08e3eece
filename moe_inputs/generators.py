"""Seeded input generators for the MoE layer workloads.

Every tensor comes from NumPy's PCG64 seeded by ``SeedSequence([seed, tag])``
so that each tensor of a workload is reproducible on its own, whatever else is
drawn. Floating tensors are drawn in float32; bf16 tensors are then rounded to
nearest-even by ``torch.Tensor.to(torch.bfloat16)`` and handed out as their
raw uint16 bit patterns, which both the GPU path (as device memory) and the
oracle (after its own decode) consume.

Value distributions:
  x, dy            ~ N(0, 1)
  router weights   ~ N(0, 1/d)               (fan-in d)
  gate, up weights ~ N(0, 1/d)               (fan-in d)
  down weights     ~ N(0, 1/F)               (fan-in F)

Routing patterns (the pages' headline rows are random-routed system benchmarks,
deniz.in, "Ai2'nin raporladığı sayılar"; the production rows use top-4,
bigchange.ai pt-BR, "O que um engenheiro pode realmente testar"):
  learned     logits are computed from x and the router weights (not here)
  uniform     each token takes k distinct experts, uniformly (first k of a
              random permutation); gate weights ~ Dirichlet(1, ..., 1)
  zipf        expert popularity proportional to rank^-s over a seeded
              permutation of the experts, with the ``zero_cold`` coldest ranks
              set to zero so that those experts receive no rows; each token
              draws k distinct experts without replacement in proportion to
              popularity (Gumbel-top-k); gate weights ~ Dirichlet(1, ..., 1)
  pregrouped  rows arrive already grouped by expert (one GPU's share of
              expert-parallel work); per-expert counts are the largest-
              remainder rounding of R * rank^-s / sum(rank^-s) over a seeded
              permutation of the experts
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

_TAGS = {
    "x": 1, "w_r": 2, "w_gate": 3, "w_up": 4, "w_down": 5, "dy": 6,
    "route_perm": 7, "route_w": 8, "zipf_perm": 9, "gumbel": 10,
    "x_perm": 11, "dy_perm": 12, "group_perm": 13,
    "w_gate_s": 14, "w_up_s": 15, "w_down_s": 16,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (for pregrouped: routed rows R)
    d: int            # model dim
    E: int            # experts
    k: int            # experts per token (pregrouped: 1)
    F: int            # expert FFN hidden dim
    dtype: str        # 'f32' | 'bf16' | 'mxfp8'
    routing: str      # 'learned' | 'uniform' | 'zipf' | 'pregrouped'
    backward: bool
    seed: int
    zipf_s: float = 0.0
    zero_cold: int = 0
    capacity_factor: float = 0.0   # > 0: padded-to-capacity comparison path
    shared_ff: int = 0             # > 0: one shared expert of this hidden size

    @property
    def R(self) -> int:
        return self.T * self.k

    def capacity(self) -> int:
        """Common per-expert capacity ceil(cf * T * k / E) of the padded path."""
        if self.capacity_factor <= 0:
            return 0
        num = round(self.capacity_factor * 1000) * self.T * self.k
        return -(-num // (1000 * self.E))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    # fp32 forward only, correctness case
    Workload("tiny_f32_fwd", T=256, d=128, E=8, k=2, F=256, dtype="f32",
             routing="learned", backward=False, seed=1),
    # small expert pool, learned router (8-expert end of the expert-pool sweep)
    Workload("e8_learned_bf16", T=16384, d=2048, E=8, k=4, F=1024, dtype="bf16",
             routing="learned", backward=True, seed=2),
    # large expert pool under uniform random routing: the headline workload
    Workload("e128_uniform_bf16", T=16384, d=2048, E=128, k=4, F=1024, dtype="bf16",
             routing="uniform", backward=True, seed=3),
    # skewed routing with a padded-to-capacity comparison (cf = 1.25)
    Workload("e128_zipf_bf16", T=16384, d=2048, E=128, k=4, F=1024, dtype="bf16",
             routing="zipf", backward=True, seed=4, zipf_s=1.2, zero_cold=8,
             capacity_factor=1.25),
    # MXFP8 one-GPU expert-parallel share, rows pre-grouped
    Workload("e32_mxfp8_share", T=32768, d=4096, E=32, k=1, F=2048, dtype="mxfp8",
             routing="pregrouped", backward=True, seed=5, zipf_s=0.8),
    # 8-expert control under the same random routing as the headline workload
    Workload("e8_uniform_bf16", T=16384, d=2048, E=8, k=4, F=1024, dtype="bf16",
             routing="uniform", backward=True, seed=3),
]}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag]])))


def _normal(seed: int, tag: str, shape, std: float) -> np.ndarray:
    a = _rng(seed, tag).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Inputs are held in the workload's storage type: float32 for 'f32',
    bf16 bit patterns (uint16) otherwise (MXFP8 operands are quantised from
    bf16 by the layer itself)."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    return _to_bf16_bits(a)


def uniform_routing(seed: int, T: int, E: int, k: int):
    keys = _rng(seed, "route_perm").random((T, E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = _rng(seed, "route_w").dirichlet(np.ones(k), size=T).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def zipf_popularity(seed: int, E: int, s: float, zero_cold: int) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p_rank = ranks ** (-s)
    if zero_cold:
        p_rank[E - zero_cold:] = 0.0
    p_rank /= p_rank.sum()
    perm = _rng(seed, "zipf_perm").permutation(E)
    p = np.empty(E)
    p[perm] = p_rank          # expert perm[r] has rank r + 1
    return p


def zipf_routing(seed: int, T: int, E: int, k: int, s: float, zero_cold: int):
    p = zipf_popularity(seed, E, s, zero_cold)
    if np.count_nonzero(p) < k:
        raise ValueError("fewer experts with non-zero popularity than k")
    g = _rng(seed, "gumbel").gumbel(size=(T, E))
    with np.errstate(divide="ignore"):
        keys = np.log(p)[None, :] + g
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = _rng(seed, "route_w").dirichlet(np.ones(k), size=T).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def pregrouped_counts(seed: int, R: int, E: int, s: float) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    share = R * ranks ** (-s) / np.sum(ranks ** (-s))
    base = np.floor(share).astype(np.int64)
    rem = R - int(base.sum())
    frac = share - base
    order = np.argsort(-frac, kind="stable")
    base[order[:rem]] += 1
    perm = _rng(seed, "group_perm").permutation(E)
    counts = np.empty(E, dtype=np.int32)
    counts[perm] = base       # expert perm[r] has rank r + 1
    return counts


def make_inputs(wl: Workload, with_weights: bool = True) -> Dict[str, np.ndarray]:
    """Inputs of one workload. Keys present depend on the routing mode:
    x [T,d] (or x_perm [R,d] and counts [E] when pregrouped), w_r [d,E]
    (learned), topk_idx [T,k] int32 and topk_w [T,k] float32 (uniform, zipf),
    w_gate, w_up [E,d,F], w_down [E,F,d], dy [T,d] (or dy_perm [R,d]); with a
    shared expert also w_gate_s, w_up_s [d,F_s] and w_down_s [F_s,d]."""
    T, d, E, k, F, s = wl.T, wl.d, wl.E, wl.k, wl.F, wl.seed
    st = "f32" if wl.dtype == "f32" else "bf16"
    out: Dict[str, np.ndarray] = {}
    if wl.routing == "pregrouped":
        out["counts"] = pregrouped_counts(s, T, E, wl.zipf_s)
        out["x_perm"] = _store(_normal(s, "x_perm", (T, d), 1.0), st)
        if wl.backward:
            out["dy_perm"] = _store(_normal(s, "dy_perm", (T, d), 1.0), st)
    else:
        out["x"] = _store(_normal(s, "x", (T, d), 1.0), st)
        if wl.backward:
            out["dy"] = _store(_normal(s, "dy", (T, d), 1.0), st)
        if wl.routing == "learned":
            out["w_r"] = _store(_normal(s, "w_r", (d, E), d ** -0.5), st)
        elif wl.routing == "uniform":
            out["topk_idx"], out["topk_w"] = uniform_routing(s, T, E, k)
        elif wl.routing == "zipf":
            out["topk_idx"], out["topk_w"] = zipf_routing(s, T, E, k, wl.zipf_s, wl.zero_cold)
        else:
            raise ValueError(wl.routing)
    if with_weights:
        out["w_gate"] = _store(_normal(s, "w_gate", (E, d, F), d ** -0.5), st)
        out["w_up"] = _store(_normal(s, "w_up", (E, d, F), d ** -0.5), st)
        out["w_down"] = _store(_normal(s, "w_down", (E, F, d), F ** -0.5), st)
        if wl.shared_ff > 0:
            Fs = wl.shared_ff
            out["w_gate_s"] = _store(_normal(s, "w_gate_s", (d, Fs), d ** -0.5), st)
            out["w_up_s"] = _store(_normal(s, "w_up_s", (d, Fs), d ** -0.5), st)
            out["w_down_s"] = _store(_normal(s, "w_down_s", (Fs, d), Fs ** -0.5), st)
    return out
