"""Pins of the oracle's router and routing metadata: hand-worked golden cases,
brute-force per-token loops, closed forms and invariants."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle.moe import expert_offsets, route, route_bwd
from oracle.numerics import round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_route(logits, k):
    T, E = logits.shape
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        pairs = sorted(((-float(logits[t, e]) + 0.0, e) for e in range(E)))
        sel = [e for _, e in pairs[:k]]
        m = max(float(logits[t, e]) for e in sel)
        ex = [math.exp(float(logits[t, e]) - m) for e in sel]
        s = sum(ex)
        idx[t] = sel
        w[t] = [v / s for v in ex]
    return idx, w


def test_route_golden_cases():
    for case in json.load(open(os.path.join(GOLDEN, "route_cases.json")))["cases"]:
        lg = round_f32(np.array([case["logits"]], dtype=np.float64))
        idx, w = route(lg, case["k"])
        assert idx[0].tolist() == case["idx"]
        np.testing.assert_allclose(w[0], case["w"], rtol=0, atol=2e-7)


def test_route_matches_brute_force_with_ties():
    rng = np.random.default_rng(0)
    # coarse values force many exact ties, including +0 and -0
    lg = rng.integers(-3, 4, size=(300, 8)).astype(np.float64) * 0.5
    lg[rng.random(lg.shape) < 0.1] = -0.0
    for k in (1, 2, 4, 8):
        idx, w = route(lg, k)
        bi, bw = _brute_route(lg, k)
        assert np.array_equal(idx, bi)
        np.testing.assert_allclose(w, bw, rtol=1e-7, atol=0)


def test_route_closed_forms():
    rng = np.random.default_rng(1)
    lg = round_f32(rng.standard_normal((64, 16)))
    idx, w = route(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    idx, w = route(lg, 16)              # k = E: a plain softmax, sorted
    sm = softmax(lg, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(sm, idx.astype(np.int64), 1), rtol=1e-6)
    # all-equal logits -> experts 0..k-1 with weight 1/k
    idx, w = route(np.zeros((4, 8)), 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (4, 1)))
    assert np.all(w == 0.25)
    # renormalised top-k of the full softmax equals softmax over selected logits
    idx, w = route(lg, 4)
    p = np.take_along_axis(sm, idx.astype(np.int64), 1)
    np.testing.assert_allclose(w, p / p.sum(1, keepdims=True), rtol=1e-6)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)


def test_route_bwd_finite_difference_and_zero_outside():
    rng = np.random.default_rng(2)
    T, E, k = 6, 8, 3
    lg = rng.standard_normal((T, E))
    dw = rng.standard_normal((T, k))
    idx, _ = route(lg, k)

    def loss(l):
        sel = np.take_along_axis(l, idx.astype(np.int64), 1)
        z = np.exp(sel - sel.max(1, keepdims=True))
        return np.sum(dw * z / z.sum(1, keepdims=True))

    w64 = softmax(np.take_along_axis(lg, idx.astype(np.int64), 1), axis=1)
    dl = route_bwd(idx, w64, dw, E)
    h = 1e-6
    fd = np.zeros_like(lg)
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += h
            lm[t, e] -= h
            fd[t, e] = (loss(lp) - loss(lm)) / (2 * h)
    np.testing.assert_allclose(dl, fd, atol=1e-6)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, 1)
    assert np.all(dl[~mask] == 0.0)


def _brute_offsets(idx, E, C):
    flat = idx.reshape(-1)
    R = flat.size
    seen = [0] * E
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    starts = [0] * (E + 1)
    for e in range(E):
        starts[e + 1] = starts[e] + counts[e]
    row_of = []
    for s in range(R):
        e = flat[s]
        r = seen[e]
        seen[e] += 1
        if C:
            row_of.append(e * C + r if r < C else -1)
        else:
            row_of.append(starts[e] + r)
    return counts, starts, row_of


@pytest.mark.parametrize("E,k,T,C", [(8, 2, 50, 0), (8, 2, 50, 9), (16, 4, 33, 0),
                                     (16, 4, 33, 5), (1, 1, 7, 0), (5, 5, 9, 0), (4, 2, 1, 0)])
def test_offsets_brute_force(E, k, T, C):
    rng = np.random.default_rng(E * 100 + k + T + C)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    m = expert_offsets(idx, E, C)
    counts, starts, row_of = _brute_offsets(idx, E, C)
    assert m["counts"].tolist() == counts
    assert m["offsets"].tolist() == starts
    assert m["row_of"].tolist() == row_of
    assert m["n_dropped"] == sum(r < 0 for r in row_of)


def test_offsets_invariants_and_stable_sort():
    rng = np.random.default_rng(5)
    T, E, k = 2000, 64, 4
    p = rng.dirichlet(np.ones(E) * 0.3)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    m = expert_offsets(idx, E)
    R = T * k
    assert m["counts"].sum() == R and m["offsets"][-1] == R
    assert np.array_equal(np.sort(m["row_of"]), np.arange(R))                 # bijection
    assert np.array_equal(m["src_slot"][m["row_of"]], np.arange(R))          # inverse
    # rows follow a stable sort of the flat expert ids (numpy's own sort)
    assert np.array_equal(m["src_slot"], np.argsort(idx.reshape(-1), kind="stable"))
    flat = idx.reshape(-1)
    assert np.all(np.diff(flat[m["src_slot"]]) >= 0)                          # expert-major


def test_offsets_padded_invariants():
    rng = np.random.default_rng(6)
    T, E, k, C = 500, 16, 4, 100
    p = np.arange(1, E + 1, dtype=float) ** -1.2
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    m = expert_offsets(idx, E, C)
    kept = np.minimum(m["counts"], C)
    assert m["n_dropped"] == int(np.sum(m["counts"] - kept))
    assert m["src_slot"].size == E * C
    for e in range(E):
        blk = m["src_slot"][e * C:(e + 1) * C]
        assert np.all(blk[:kept[e]] >= 0) and np.all(blk[kept[e]:] == -1)
        assert np.all(np.diff(blk[:kept[e]]) > 0)                              # slot order
        assert np.all(idx.reshape(-1)[blk[:kept[e]]] == e)
    # a dropped slot of expert e comes after all of e's kept slots
    flat = idx.reshape(-1)
    for s in np.nonzero(m["row_of"] < 0)[0]:
        e = flat[s]
        assert s > m["src_slot"][e * C + C - 1]


def test_router_logits_special_cases():
    """The learned router's logits x . W_r [d, E] in binary32: a one-hot
    token row picks out one row of W_r exactly; small-integer operands give
    exact dot products that a per-element loop reproduces; each logit is
    linear in the token and the result is [T, E] (a transposed operand or a
    dropped term fails one of these)."""
    from oracle.moe import router_logits
    rng = np.random.default_rng(30)
    d, E = 12, 5
    w_r = rng.standard_normal((d, E)).astype(np.float32).astype(np.float64)
    eye = np.eye(d)
    assert np.array_equal(router_logits(eye, w_r), w_r)                 # one-hot rows
    assert router_logits(eye[:3], w_r).shape == (3, E)
    xi = rng.integers(-4, 5, size=(7, d)).astype(np.float64)
    wi = rng.integers(-4, 5, size=(d, E)).astype(np.float64)
    brute = np.array([[sum(xi[t, i] * wi[i, e] for i in range(d)) for e in range(E)] for t in range(7)])
    assert np.array_equal(router_logits(xi, wi), brute)
    x = rng.standard_normal((4, d))
    lhs = router_logits(2.0 * x[:1] + x[1:2], w_r)[0]
    rhs = 2.0 * (x[0] @ w_r) + x[1] @ w_r
    assert np.allclose(lhs, rhs, rtol=1e-6, atol=1e-6)
    # stored in binary32
    assert np.array_equal(router_logits(x, w_r), router_logits(x, w_r).astype(np.float32))
