"""Host-side logic of the layer classes that needs no GPU."""
import gc

import torch

from routing_grouped_expert_router_amd.mx_layer import WeightVersion


def test_weight_version_requantises_on_write_or_new_tensor():
    """The MXFP8 experts keep quantised weight copies only while the same
    weight tensors come back unmodified: an in-place write, or a new tensor
    (even one that reuses the freed tensor's memory), must requantise."""
    ws = [torch.randn(4, 8, 16) for _ in range(3)]
    v = WeightVersion()
    assert not v.matches(ws)
    v.record(ws)
    assert v.matches(ws)
    assert not v.matches(ws[:2])
    ws[1].add_(1.0)                       # an optimiser step, in place
    assert not v.matches(ws)
    v.record(ws)
    assert v.matches(ws)
    # a freed weight replaced by a fresh tensor of the same shape: the caching
    # allocator may hand back the very same block
    addr = ws[0].data_ptr()
    ws[0] = None
    gc.collect()
    fresh = torch.empty(4, 8, 16)
    fresh.copy_(torch.randn(4, 8, 16))
    ws[0] = fresh
    assert not v.matches(ws), f"reused address {addr == fresh.data_ptr()}"
    # a view of the same storage is another tensor object: requantise too
    v.record(ws)
    assert not v.matches([ws[0].view(4, 8, 16), ws[1], ws[2]])
    v.clear()
    assert not v.matches(ws)
