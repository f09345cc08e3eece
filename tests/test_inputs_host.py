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
