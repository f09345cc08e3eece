"""Every kernel of libmoe compiles without scratch memory or register spills.

A wave's private (scratch) memory goes through the vector memory path; in a
memory-bound kernel a spill, or a select of whole vectors that the compiler
lowers through a stack slot, costs far more than the registers it saves (a
router kernel ran at a third of its rate that way). The build writes the
compiler's per-kernel resource remarks next to the objects; this reads them,
building first when they are missing.
"""
import os

from routing_grouped_expert_router_amd import build as b


def _reports():
    srcs = b.sources()
    if not all(os.path.exists(b.resource_report(s)) for s in srcs):
        b.build()
    return {os.path.basename(s): b.parse_resources(open(b.resource_report(s)).read()) for s in srcs}


def test_no_scratch_and_no_spills():
    reports = _reports()
    kernels = 0
    for src, kern in reports.items():
        for name, f in kern.items():
            kernels += 1
            assert f.get("ScratchSize [bytes/lane]") == "0", (src, name, f)
            assert f.get("VGPRs Spill") == "0" and f.get("SGPRs Spill") == "0", (src, name, f)
    # the report covers every source and the library's hot kernels
    assert set(reports) == {os.path.basename(s) for s in b.sources()}
    names = " ".join(n for k in reports.values() for n in k)
    for hot in ("gg_dma_kernel", "gg_mx_kernel", "mx_both_kernel", "permute_kernel", "combine_bwd_rows_kernel",
                "router_gemm_mfma_kernel", "router_bwd_mfma_kernel"):
        assert hot in names, hot
    assert kernels > 40
