"""CPU oracle for one MoE layer's forward and backward pass.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, float64 statement
of what the layer computes. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the GPU path never does, and
it imports nothing from the GPU path.

Sources. The pages describe Ai2's Olmo-core 3 MoE training stack in prose:
  * sparse top-k MoE, each token visits a few experts
    (deniz.in, "Hedeflediği kapasite sorunu");
  * routing metadata (split and group sizes) kept on the GPU
    (deniz.in, "Yeni stack nasıl çalışıyor"; unite.ai/hi,
    "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें");
  * selected token rows written straight into the expert's input buffer
    (same sections; donmalab.com, "擴展與最佳化手段");
  * grouped GEMMs over the uneven per-expert shapes, measured against
    padding every group to a common capacity (deniz.in, "Yeni stack nasıl
    çalışıyor");
  * MXFP8 for the feed-forward GEMMs (bigchange.ai pt-BR, "Três números,
    três denominadores"; unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन, और मेमोरी
    तकनीकें").
The pages give no formula. Where they are silent the oracle takes the plainest
reading (softmax router with top-k and renormalisation, SwiGLU experts,
stable expert-major row order, ceil-capacity with overflow dropped in slot
order, OCP MX v1.0 for MXFP8); each function states its reading.

Pins. Every function here is checked by the CPU tests against something other
than itself: brute-force per-token loops, closed forms, invariants, adjoint
identities, central finite differences, torch's own bf16/float8 casts and the
OCP format tables. No function is parity-unpinned.
"""
