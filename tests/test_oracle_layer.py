"""Pins of the oracle's layer: brute-force per-token expert loops, the dense
special case, the identical-experts invariant, padded/dropless agreement,
adjoint identities and central finite differences of the whole backward."""
import numpy as np
import pytest

import oracle.moe as om
from oracle.moe import (
    combine, combine_bwd, expert_offsets, layer_backward, layer_forward, permute,
    permute_bwd, route,
)
from oracle.numerics import round_bf16, round_f32


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _params(rng, T, d, E, F, learned=True, k=2):
    p = {
        "x": rng.standard_normal((T, d)),
        "w_gate": rng.standard_normal((E, d, F)) / np.sqrt(d),
        "w_up": rng.standard_normal((E, d, F)) / np.sqrt(d),
        "w_down": rng.standard_normal((E, F, d)) / np.sqrt(F),
    }
    if learned:
        p["w_r"] = rng.standard_normal((d, E)) / np.sqrt(d)
    else:
        p["topk_idx"] = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        p["topk_w"] = rng.dirichlet(np.ones(k), size=T)
    return p


def _token_loop(p, k):
    """y[t] = sum_j w_j FFN_{e_j}(x[t]) one token at a time, no permutation."""
    T = p["x"].shape[0]
    y = np.zeros_like(p["x"])
    for t in range(T):
        xt = p["x"][t]
        if "w_r" in p:
            lg = xt @ p["w_r"]
            sel = sorted(range(lg.size), key=lambda e: (-lg[e], e))[:k]
            z = np.exp(lg[sel] - lg[sel].max())
            w = z / z.sum()
        else:
            sel, w = p["topk_idx"][t], p["topk_w"][t]
        for j, e in enumerate(sel):
            h = _silu(xt @ p["w_gate"][e]) * (xt @ p["w_up"][e])
            y[t] += w[j] * (h @ p["w_down"][e])
    return y


@pytest.mark.parametrize("learned", [True, False])
def test_forward_matches_token_loop(learned):
    rng = np.random.default_rng(10)
    T, d, E, F, k = 40, 16, 8, 24, 2
    p = _params(rng, T, d, E, F, learned, k)
    if learned:
        # route with unrounded float64 logits so the loop's selection is identical
        lg = p["x"] @ p["w_r"]
        fwd = layer_forward(p, k, "f64", logits=lg)
    else:
        fwd = layer_forward(p, k, "f64")
    np.testing.assert_allclose(fwd["y"], _token_loop(p, k), rtol=0, atol=1e-12)


def test_single_expert_is_dense_ffn():
    rng = np.random.default_rng(11)
    p = _params(rng, 17, 8, 1, 12, learned=True)
    fwd = layer_forward(p, 1, "f64")
    assert np.all(fwd["topk_w"] == 1.0)
    x = p["x"]
    dense = (_silu(x @ p["w_gate"][0]) * (x @ p["w_up"][0])) @ p["w_down"][0]
    np.testing.assert_allclose(fwd["y"], dense, rtol=0, atol=1e-12)


def test_identical_experts_invariant():
    """With every expert holding the same weights, y = FFN(x) whatever the
    routing, because the gate weights of a token sum to one."""
    rng = np.random.default_rng(12)
    T, d, E, F, k = 64, 16, 8, 20, 4
    p = _params(rng, T, d, E, F, learned=True)
    for name in ("w_gate", "w_up", "w_down"):
        p[name][:] = p[name][0]
    fwd = layer_forward(p, k, "f64")
    x = p["x"]
    dense = (_silu(x @ p["w_gate"][0]) * (x @ p["w_up"][0])) @ p["w_down"][0]
    np.testing.assert_allclose(fwd["y"], dense, rtol=1e-6, atol=1e-6)   # w are binary32
    np.testing.assert_allclose(fwd["topk_w"].sum(1), 1.0, atol=1e-6)


def test_padded_equals_dropless_when_nothing_drops():
    rng = np.random.default_rng(13)
    T, d, E, F, k = 96, 16, 8, 16, 2
    p = _params(rng, T, d, E, F, learned=False, k=k)
    for n in ("x", "w_gate", "w_up", "w_down"):
        p[n] = round_bf16(p[n])
    dy = round_bf16(rng.standard_normal((T, d)))
    a = layer_forward(p, k, "bf16")
    C = int(a["counts"].max()) + 3
    b = layer_forward(p, k, "bf16", capacity=C)
    assert b["n_dropped"] == 0
    assert np.array_equal(a["y"], b["y"])
    ga = layer_backward(p, a, dy, k, "bf16")
    gb = layer_backward(p, b, dy, k, "bf16", capacity=C)
    for name in ("dx", "dw_gate", "dw_up", "dw_down", "dtopk_w"):
        assert np.array_equal(ga[name], gb[name]), name


def test_adjoint_identities():
    rng = np.random.default_rng(14)
    T, d, E, k = 30, 12, 6, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    f64 = lambda a: a
    for C in (0, 4):
        m = expert_offsets(idx, E, C)
        x = rng.standard_normal((T, d))
        u = rng.standard_normal((m["n_rows"], d))
        u[m["src_slot"] < 0] = 0.0
        lhs = np.sum(permute(x, m["src_slot"], k) * u)
        rhs = np.sum(x * permute_bwd(u, m["row_of"], T, k, f64))
        assert abs(lhs - rhs) <= 1e-11 * (1 + abs(lhs))
        Y = rng.standard_normal((m["n_rows"], d))
        w = rng.random((T, k))
        v = rng.standard_normal((T, d))
        dyp, dw = combine_bwd(v, Y, w, m["row_of"], m["n_rows"], f64)
        lhs = np.sum(combine(Y, m["row_of"], w, T, k, f64) * v)
        assert abs(lhs - np.sum(Y * dyp)) <= 1e-11 * (1 + abs(lhs))
        # combine is linear in w too: <combine(Y; w'), v> = <w', dw> (dw in binary32)
        w2 = rng.random((T, k))
        lhs = np.sum(combine(Y, m["row_of"], w2, T, k, f64) * v)
        assert abs(lhs - np.sum(w2 * dw)) <= 1e-5 * (1 + abs(lhs))


def _fd_check(p, k, capacity, names, seed):
    rng = np.random.default_rng(seed)
    T, d = p["x"].shape
    dy = rng.standard_normal((T, d))
    fwd = layer_forward(p, k, "f64", capacity=capacity,
                        logits=(p["x"] @ p["w_r"]) if "w_r" in p else None)
    g = layer_backward(p, fwd, dy, k, "f64", capacity=capacity)
    gmap = {"x": "dx", "w_gate": "dw_gate", "w_up": "dw_up", "w_down": "dw_down", "w_r": "dw_r",
            "w_gate_s": "dw_gate_s", "w_up_s": "dw_up_s", "w_down_s": "dw_down_s"}

    def loss(q):
        f = layer_forward(q, k, "f64", capacity=capacity,
                          logits=(q["x"] @ q["w_r"]) if "w_r" in q else None)
        assert np.array_equal(f["topk_idx"], fwd["topk_idx"])       # routing frozen
        return np.sum(f["y"] * dy)

    h = 1e-6
    for name in names:
        arr = p[name]
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            q = {kk: vv.copy() for kk, vv in p.items()}
            q[name][i] += h
            lp = loss(q)
            q[name][i] -= 2 * h
            lm = loss(q)
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gmap[name]], fd, rtol=1e-5, atol=1e-7, err_msg=name)


def test_backward_finite_differences_learned_router():
    rng = np.random.default_rng(15)
    T, d, E, F, k = 8, 16, 4, 32, 2
    p = _params(rng, T, d, E, F, learned=True)
    lg = p["x"] @ p["w_r"]
    srt = -np.sort(-lg, axis=1)
    assert np.min(srt[:, k - 1] - srt[:, k]) > 1e-3       # no selection flips under FD
    _fd_check(p, k, 0, ["x", "w_r", "w_gate", "w_up", "w_down"], 16)


def test_backward_finite_differences_padded_with_drops():
    rng = np.random.default_rng(17)
    T, d, E, F, k = 10, 8, 4, 12, 2
    p = _params(rng, T, d, E, F, learned=False, k=k)
    m = expert_offsets(p["topk_idx"], E, 3)
    assert m["n_dropped"] > 0
    _fd_check(p, k, 3, ["x", "w_gate", "w_up", "w_down"], 18)


def _with_shared(rng, p, F_s):
    d = p["x"].shape[1]
    p["w_gate_s"] = rng.standard_normal((d, F_s)) / np.sqrt(d)
    p["w_up_s"] = rng.standard_normal((d, F_s)) / np.sqrt(d)
    p["w_down_s"] = rng.standard_normal((F_s, d)) / np.sqrt(F_s)
    return p


def test_shared_expert_finite_differences():
    rng = np.random.default_rng(19)
    T, d, E, F, k = 8, 12, 4, 16, 2
    p = _with_shared(rng, _params(rng, T, d, E, F, learned=False, k=k), 20)
    _fd_check(p, k, 0, ["x", "w_gate_s", "w_up_s", "w_down_s"], 20)


def test_shared_expert_equals_a_routed_expert_every_token_takes():
    # one routed expert taken by every token with gate weight 1 and no shared
    # expert, against a routed expert that outputs zero plus a shared expert
    # with the same weights: forward and every gradient agree exactly
    rng = np.random.default_rng(21)
    T, d, F = 24, 16, 20
    a = _params(rng, T, d, 1, F, learned=False, k=1)
    a["topk_w"] = np.ones((T, 1))
    b = {n: v.copy() for n, v in a.items()}
    b["w_gate_s"], b["w_up_s"], b["w_down_s"] = a["w_gate"][0], a["w_up"][0], a["w_down"][0]
    b["w_down"] = np.zeros_like(a["w_down"])
    dy = rng.standard_normal((T, d))
    fa, fb = layer_forward(a, 1, "f64"), layer_forward(b, 1, "f64")
    assert np.array_equal(fa["y"], fb["y"])
    ga, gb = layer_backward(a, fa, dy, 1, "f64"), layer_backward(b, fb, dy, 1, "f64")
    assert np.array_equal(ga["dx"], gb["dx"])
    for n in ("w_gate", "w_up", "w_down"):
        assert np.array_equal(ga["d" + n][0], gb["d" + n + "_s"]), n


def test_fp32_storage_is_close_to_f64():
    rng = np.random.default_rng(19)
    p = _params(rng, 32, 16, 4, 24, learned=True)
    a = layer_forward(p, 2, "f64", logits=round_f32(p["x"] @ p["w_r"]))
    b = layer_forward(p, 2, "f32")
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(b["y"], a["y"], rtol=0, atol=1e-6 * np.abs(a["y"]).max())


# ----------------------------------------------------------------------------- MXFP8
def _mx_inputs(rng, counts, d, F):
    E = len(counts)
    n = int(np.sum(counts))
    q = lambda a: round_bf16(a)
    return (q(rng.standard_normal((n, d))), q(rng.standard_normal((n, d))),
            np.asarray(counts), q(rng.standard_normal((E, d, F)) / np.sqrt(d)),
            q(rng.standard_normal((E, d, F)) / np.sqrt(d)),
            q(rng.standard_normal((E, F, d)) / np.sqrt(F)))


def test_mx_layer_without_quantisation_is_the_bf16_layer(monkeypatch):
    """With the MX round trip replaced by the identity, the MX expert layer is
    exactly the bf16 expert chain on the same grouped rows."""
    rng = np.random.default_rng(20)
    counts = [5, 0, 40, 33]
    xp, dyp, counts, wg, wu, wd = _mx_inputs(rng, counts, 64, 96)
    monkeypatch.setattr(om, "mx_roundtrip", lambda a: np.asarray(a, dtype=np.float64))
    out = om.mx_expert_layer(xp, dyp, counts, wg, wu, wd)
    st = round_bf16
    off = np.concatenate([[0], np.cumsum(counts)])
    groups = [(int(off[e]), int(counts[e])) for e in range(len(counts))]
    G, U, H = om.expert_fwd_gate_up(xp, wg, wu, groups, st)
    Y = om.expert_fwd_down(H, wd, groups, st)
    dG, dU = om.expert_dgrad_down(dyp, wd, G, U, groups, st)
    dX = om.expert_dgrad_gate_up(dG, dU, wg, wu, groups, st)
    dWd = om.expert_wgrad_down(H, dyp, groups, 96, 64, st)
    dWg, dWu = om.expert_wgrad_gate_up(xp, dG, dU, groups, 64, 96, st)
    for name, ref in dict(G=G, U=U, H=H, y_perm=Y, dG=dG, dU=dU, dx_perm=dX,
                          dw_gate=dWg, dw_up=dWu, dw_down=dWd).items():
        assert np.array_equal(out[name], ref), name


def test_mx_layer_blocks_run_along_each_contraction(monkeypatch):
    """Every quantised operand is blocked along the contraction axis of the
    GEMM it feeds: the model dim (64), the hidden dim (96) or the expert's own
    rows (40 or 33), never anything else."""
    rng = np.random.default_rng(21)
    counts = [40, 33]
    args = _mx_inputs(rng, counts, 64, 96)
    seen = []

    def spy(a):
        a = np.asarray(a, dtype=np.float64)
        seen.append(a.shape)
        return a
    monkeypatch.setattr(om, "mx_roundtrip", spy)
    om.mx_expert_layer(*args)
    # per expert: fwd X, Wg^T, Wu^T, H, Wd^T; dgrad dY, Wd; dG, Wg, dU, Wu;
    # wgrad H^T, dY^T, X^T, dG^T, dU^T
    want = []
    for n in counts:
        want += [(n, 64), (96, 64), (96, 64), (n, 96), (64, 96), (n, 64), (96, 64),
                 (n, 96), (64, 96), (n, 96), (64, 96), (96, n), (64, n), (64, n), (96, n), (96, n)]
    assert seen == want


def test_mx_layer_error_against_bf16_layer():
    rng = np.random.default_rng(22)
    counts = [37, 64, 3]
    xp, dyp, counts, wg, wu, wd = _mx_inputs(rng, counts, 64, 96)
    mx = om.mx_expert_layer(xp, dyp, counts, wg, wu, wd)
    off = np.concatenate([[0], np.cumsum(counts)])
    groups = [(int(off[e]), int(counts[e])) for e in range(len(counts))]
    st = round_bf16
    G, U, H = om.expert_fwd_gate_up(xp, wg, wu, groups, st)
    Y = om.expert_fwd_down(H, wd, groups, st)
    rel = np.abs(mx["y_perm"] - Y).max() / np.abs(Y).max()
    assert 1e-4 < rel < 0.1


def test_mx_routed_layer_without_quantisation_is_the_bf16_layer(monkeypatch):
    # with the quantiser replaced by the identity, the MXFP8 routed layer must
    # be the bf16 layer exactly (routing, permute, combine and adjoints are
    # shared; only the expert GEMM operands are quantised)
    rng = np.random.default_rng(22)
    T, d, E, F, k = 40, 64, 6, 96, 2
    for learned in (False, True):
        p = _params(rng, T, d, E, F, learned=learned, k=k)
        for n in list(p):
            if n.startswith("w_") or n == "x":
                p[n] = round_bf16(p[n])
        dy = round_bf16(rng.standard_normal((T, d)))
        monkeypatch.setattr(om, "mx_roundtrip", lambda a: np.asarray(a, dtype=np.float64))
        mx = om.mx_layer(p, k, dy)
        monkeypatch.undo()
        fwd = layer_forward(p, k, "bf16")
        bwd = layer_backward(p, fwd, dy, k, "bf16")
        for n in ("y",):
            assert np.array_equal(mx[n], fwd[n]), n
        for n in ("dx", "dw_gate", "dw_up", "dw_down", "dtopk_w", "dy_perm"):
            ref = bwd[n]
            assert np.array_equal(mx[n], ref), n
        if learned:
            assert np.array_equal(mx["dw_r"], bwd["dw_r"])
