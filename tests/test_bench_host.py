"""Host-side checks of the measurement plumbing: the committed rocprofv3
summaries parse, kernel names map to pipeline stages, and the algorithmic
byte counts add up."""
import glob
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_summaries_parse():
    from profile_summary import read_traffic_table
    files = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))
    assert files, "no traffic summary under profiles/"
    for f in files:
        tab = read_traffic_table(f)
        wl = os.path.basename(f)[len("traffic_"):-3]
        assert wl in tab
        for st, ent in tab[wl].items():
            assert ent["bytes_per_launch"] > 0 and len(ent["source_hash"]) == 16


@pytest.mark.parametrize("name,stage", [
    ("void moe::gg_dma_kernel<0, moe::DmaCfg<128, 256, 2, 2, 32, 3, 2> >(moe::GGArgs)", "gg_fwd_gate_up"),
    ("void moe::gg_dma_kernel<5, moe::DmaCfg<128, 256, 2, 2, 32, 3, 2> >(moe::GGArgs)", "gg_wgrad_gate_up"),
    ("void moe::combine_bwd_kernel<unsigned short>(unsigned short const*)", "combine_bwd"),
    ("void moe::combine_kernel<unsigned short>(unsigned short const*)", "combine"),
    ("moe::scan_kernel(int*, int, int, int, int*, int*, int*)", "offsets"),
    ("__amd_rocclr_copyBuffer", None),
])
def test_stage_of(name, stage):
    from profile_summary import stage_of
    assert stage_of(name) == stage


def test_algorithmic_bytes():
    from bench import stage_algorithmic_bytes
    from moe_inputs import workload
    wl = workload("e128_uniform_bf16")
    R = wl.T * wl.k
    W = wl.E * wl.d * wl.F * 2
    # forward gate/up reads x_perm and both weights, writes G, U and H
    assert stage_algorithmic_bytes("gg_fwd_gate_up", wl, R, R) == R * wl.d * 2 + 2 * W + 3 * R * wl.F * 2
    # the weight gradient of the down projection writes exactly one weight tensor
    assert stage_algorithmic_bytes("gg_wgrad_down", wl, R, R) - W == R * (wl.d + wl.F) * 2


@pytest.mark.parametrize("name,stage", [
    ("void moe::gg_mx_kernel<2, moe::MxCfg<128, 256, 2, 4, 3, 2> >(moe::MxArgs)", "mx_dgrad_down"),
    ("void moe::gg_mx_kernel<5, moe::MxCfg<128, 256, 2, 4, 3, 2> >(moe::MxArgs)", "mx_wgrad_gate_up"),
    ("moe::(anonymous namespace)::mx_both_kernel(unsigned short const*, int)", "mx_quantize"),
    ("void moe::permute_bwd_kernel<unsigned short>(unsigned short const*)", "permute_bwd"),
])
def test_stage_of_mxfp8_and_adjoints(name, stage):
    from profile_summary import stage_of
    assert stage_of(name) == stage


def test_timed_means_leave_out_warmup_launches(tmp_path):
    """The kernel summary's timed mean drops each kernel's first launches
    (the traced run's warm-up steps) in launch order, whatever order the
    trace lists them in."""
    from profile_summary import _timed_means
    rows = [("k_a", 300, 400), ("k_a", 100, 190), ("k_b", 150, 160), ("k_a", 500, 520),
            ("k_a", 700, 730), ("k_b", 800, 830)]   # (name, start ns, end ns)
    path = tmp_path / "kt_kernel_trace.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, s, e in rows:
            f.write(f"{n},{s},{e}\n")
    m = _timed_means(str(path), 2)
    # k_a launches in time order last 90, 100, 20, 30 ns: the last two remain
    assert m["k_a"] == pytest.approx(25e-3)
    # k_b has only two launches: all are kept rather than none
    assert m["k_b"] == pytest.approx(20e-3)
