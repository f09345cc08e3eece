"""The no-allocation routing-metadata entry point against the allocating
one, through the C ABI: bit-identical outputs on two calls in a row, the
second with a smaller input (the static array keeps the first call's
contents), dropless and padded."""
import numpy as np
import pytest
import torch

from routing_grouped_expert_router_amd import _lib as L

pytestmark = pytest.mark.gpu


def _meta(T, k, E, capacity):
    n_rows = E * capacity if capacity > 0 else T * k
    i32 = lambda *s: torch.full(s, -7, dtype=torch.int32, device="cuda")
    return dict(counts=i32(E), offsets=i32(E + 1), row_of=i32(T * k), src_slot=i32(n_rows),
                n_dropped=i32(1), err_flag=torch.zeros(1, dtype=torch.int32, device="cuda"))


def _ids(T, k, E, seed, bad=0):
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if bad:
        idx.view(-1)[:bad] = E + 3                      # ids outside [0, E) raise the flag
    return idx.cuda()


@pytest.mark.parametrize("capacity", [0, 5])
def test_offsets_noalloc_matches_offsets(capacity):
    E = 64
    for T, k, seed, bad in ((20000, 4, 1, 0), (333, 3, 2, 7)):   # second call smaller
        cap = capacity if capacity == 0 else max(1, (capacity * T * k) // (E * 4))
        idx = _ids(T, k, E, seed, bad)
        ref, got = _meta(T, k, E, cap), _meta(T, k, E, cap)
        ws = torch.empty(L.moe_offsets_workspace_bytes(T, k, E) // 4 + 4, dtype=torch.int32, device="cuda")
        L.moe_offsets(idx, E, cap, ref["counts"], ref["offsets"], ref["row_of"], ref["src_slot"],
                      ref["n_dropped"], ref["err_flag"], ws)
        L.moe_offsets_noalloc(idx, E, cap, got["counts"], got["offsets"], got["row_of"], got["src_slot"],
                              got["n_dropped"], got["err_flag"])
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(ref[n], got[n]), (T, n)
        assert int(got["err_flag"][0]) == (1 if bad else 0)
        assert int(got["offsets"][-1]) == T * k - bad
