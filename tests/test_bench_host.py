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
    ("moe::rank_kernel(int const*, int, int, int, int const*, int, int*, int*, int*, int*, int*)", "offsets"),
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
    ("void moe::combine_bwd_rows_kernel<unsigned short>(unsigned short const*)", "combine_bwd"),
    ("void moe::gg_mx_wgrad_split_kernel<5, moe::MxCfg<128, 256, 2, 4, 3, 2> >(moe::GGArgs, int, int*)",
     "mx_wgrad_gate_up"),
    ("void moe::gg_wgrad_split_kernel<4, moe::DmaCfg<128, 256, 2, 4, 32, 3, 2> >(moe::GGArgs, int, int*)",
     "gg_wgrad_down"),
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


def test_sync_summary_flags_blocking_calls_inside_steps_only(tmp_path):
    """The host-synchronisation summary counts a blocking call or a
    device-to-host copy when it falls inside a layer step, not between steps."""
    import argparse
    from profile_summary import syncs
    hist = "void moe::hist_kernel(int const*)"
    gemm = "void moe::gg_dma_kernel<5, moe::DmaCfg<128, 256, 2, 4, 32, 3, 2> >(moe::GGArgs)"
    # (name, correlation id, GPU start, GPU end); host launch calls at 10 * id
    kern = [(hist, 1, 1000, 1100), (gemm, 2, 1200, 2000), (hist, 5, 3000, 3100), (gemm, 7, 3200, 4000)]
    api = [("hipLaunchKernel", 1, 10, 11), ("hipLaunchKernel", 2, 20, 21),
           ("hipDeviceSynchronize", 3, 30, 31),               # between the steps: allowed
           ("hipLaunchKernel", 5, 50, 51), ("hipStreamSynchronize", 6, 60, 61),   # inside step 1
           ("hipLaunchKernel", 7, 70, 71)]
    with open(tmp_path / "t_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Correlation_Id,Start_Timestamp,End_Timestamp\n")
        for n, c, a, b in kern:
            f.write(f'"{n}",{c},{a},{b}\n')
    with open(tmp_path / "t_hip_api_trace.csv", "w") as f:
        f.write("Function,Correlation_Id,Start_Timestamp,End_Timestamp\n")
        for n, c, a, b in api:
            f.write(f"{n},{c},{a},{b}\n")
    with open(tmp_path / "t_memory_copy_trace.csv", "w") as f:
        f.write("Direction,Start_Timestamp,End_Timestamp\n")
        f.write("MEMORY_COPY_DEVICE_TO_HOST,1500,1600\n")       # during step 0's GPU span
        f.write("MEMORY_COPY_DEVICE_TO_HOST,2500,2600\n")       # between the steps
    out = tmp_path / "s.md"
    bad = syncs(argparse.Namespace(out=str(out), dir=str(tmp_path), command=None, warmup=0))
    assert bad == 2
    text = out.read_text()
    assert "| 0 | 2 |" in text and "| 1 | 2 |" in text


def test_mfma_summary(tmp_path):
    """The matrix-core summary averages MfmaUtil over launches and turns MFMA
    ops into flops (512 per op) against the stage's algorithmic flops."""
    import argparse
    from profile_summary import mfma
    k = "void moe::gg_dma_kernel<1, moe::DmaCfg<128, 256, 2, 4, 32, 3, 2> >(moe::GGArgs)"
    split = "void moe::gg_wgrad_split_kernel<4, moe::DmaCfg<128, 256, 2, 4, 32, 3, 2> >(moe::GGArgs, int, int*)"
    flops = 2 * 16384 * 4 * 2048 * 1024          # forward down projection at the headline size
    with open(tmp_path / "m.csv", "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for util in (30.0, 50.0):
            f.write(f'"{k}",MfmaUtil,{util}\n"{k}",SQ_INSTS_VALU_MFMA_MOPS_BF16,{flops * 1.5 / 512}\n')
        f.write(f'"{split}",MfmaUtil,0.0\n')
    out = tmp_path / "m.md"
    mfma(argparse.Namespace(out=str(out), csv=str(tmp_path / "m.csv"), workload="e128_uniform_bf16",
                            command=None))
    line = [l for l in out.read_text().splitlines() if l.startswith("| gg_fwd_down")][0]
    assert line == "| gg_fwd_down | 2 | 40.0 | 412.3 | 274.9 | 1.500 |"
    assert "gg_wgrad_down" not in out.read_text()
    # warm-up launches left out: only the second launch counts
    mfma(argparse.Namespace(out=str(out), csv=str(tmp_path / "m.csv"), workload="e128_uniform_bf16",
                            command=None, skip=1))
    line = [l for l in out.read_text().splitlines() if l.startswith("| gg_fwd_down")][0]
    assert line == "| gg_fwd_down | 1 | 50.0 | 412.3 | 274.9 | 1.500 |"

