"""The seeded input generators: shapes, reproducibility and the stated
distributions of every tensor a workload can ask for."""
import numpy as np

from moe_inputs import make_inputs, workload
from oracle.numerics import bf16_bits_to_f64


def test_shared_expert_weights():
    wl = workload("e128_uniform_bf16").scaled(T=256, E=8, d=256, F=128, shared_ff=384)
    a, b = make_inputs(wl), make_inputs(wl)
    for n, shape, fan_in in (("w_gate_s", (256, 384), 256), ("w_up_s", (256, 384), 256),
                             ("w_down_s", (384, 256), 384)):
        assert a[n].shape == shape and a[n].dtype == np.uint16
        assert np.array_equal(a[n], b[n])                    # seeded
        v = bf16_bits_to_f64(a[n])
        assert abs(v.std() * np.sqrt(fan_in) - 1.0) < 0.02   # N(0, 1/fan_in)
    assert not np.array_equal(a["w_gate_s"], a["w_up_s"])   # distinct streams
    assert "w_gate_s" not in make_inputs(wl.scaled(shared_ff=0))


def _routing_checks(idx, w, E, k):
    T = idx.shape[0]
    assert idx.shape == (T, k) and idx.dtype == np.int32 and w.shape == (T, k) and w.dtype == np.float32
    assert idx.min() >= 0 and idx.max() < E
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "k distinct experts per token"
    assert np.all(w > 0)
    assert np.abs(w.astype(np.float64).sum(axis=1) - 1.0).max() < 1e-6   # Dirichlet draws sum to one


def test_uniform_routing_generator():
    """Headline workload: k distinct experts uniformly per token, Dirichlet(1)
    gate weights; expert loads close to T*k/E = 512 (this seed: 455..573)."""
    wl = workload("e128_uniform_bf16")
    inp = make_inputs(wl, with_weights=False)
    idx, w = inp["topk_idx"], inp["topk_w"]
    _routing_checks(idx, w, wl.E, wl.k)
    counts = np.bincount(idx.reshape(-1), minlength=wl.E)
    assert counts.sum() == wl.T * wl.k
    assert (counts.min(), counts.max()) == (455, 573)
    # Dirichlet(1, ..., 1): every weight marginal is Beta(1, k-1), mean 1/k
    assert abs(w.mean() - 1 / wl.k) < 1e-6 and abs(w[:, 0].mean() - 1 / wl.k) < 0.01
    assert np.array_equal(make_inputs(wl, with_weights=False)["topk_idx"], idx)   # seeded


def test_zipf_routing_generator():
    """Skewed workload: popularity proportional to rank^-1.2 with the 8 coldest
    ranks at zero, so exactly 8 experts receive no rows; the hottest expert
    gets far more than 3000 rows, and many slots overflow capacity 640."""
    wl = workload("e128_zipf_bf16")
    inp = make_inputs(wl, with_weights=False)
    idx, w = inp["topk_idx"], inp["topk_w"]
    _routing_checks(idx, w, wl.E, wl.k)
    counts = np.bincount(idx.reshape(-1), minlength=wl.E)
    assert (counts == 0).sum() == 8
    assert counts.max() == 12315 and counts.max() > 3000
    assert wl.capacity() == 640
    dropped = np.maximum(counts - wl.capacity(), 0).sum()
    assert dropped == 35612
    # the rank order of the non-empty experts follows the popularity order
    from moe_inputs.generators import zipf_popularity
    p = zipf_popularity(wl.seed, wl.E, wl.zipf_s, wl.zero_cold)
    assert np.array_equal(np.nonzero(p == 0)[0], np.nonzero(counts == 0)[0])
    hot = np.argsort(-p)[:8]
    assert np.all(counts[hot[:-1]] > counts[hot[1:]] * 0.9)


def test_pregrouped_counts_generator():
    """MXFP8 share: largest-remainder rounding of R * rank^-0.8 / H over a
    seeded expert permutation: sum R, min 366, max 5858; the groups are ragged
    (31 of 32 counts are not a multiple of the 32-value MX block)."""
    wl = workload("e32_mxfp8_share")
    from moe_inputs.generators import pregrouped_counts
    c = pregrouped_counts(wl.seed, wl.T, wl.E, wl.zipf_s)
    assert c.sum() == 32768 and c.min() == 366 and c.max() == 5858
    assert np.count_nonzero(c % 32) == 31
    ranks = np.arange(1, wl.E + 1, dtype=np.float64)
    share = 32768 * ranks ** -0.8 / np.sum(ranks ** -0.8)
    assert np.all(np.abs(np.sort(c)[::-1] - share) < 1.0)   # each within one of its exact share
    assert np.array_equal(make_inputs(wl.scaled(d=256), with_weights=False)["counts"], c)
