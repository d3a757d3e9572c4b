"""The allocation-free dispatch (moe_dispatch_noalloc, workspace in the
library's fixed scratch) against moe_dispatch with a caller workspace: counts,
offsets, the layout map and the gathered rows, bit for bit, on calls in a
row that reuse the scratch, each smaller than the one before: the
histogram/scan/slots path past 256 tiles, the histogram + table path, and a
one-tile batch."""

import pytest
import torch

from combine_moe_route_02_amd import _lib as L
from tests.harness import say

pytestmark = pytest.mark.gpu

CALLS = [(70000, 64, 2, 16, 48), (16384, 256, 8, 0, 32), (300, 256, 8, 0, 32)]


def _inputs(T, E, k, seed):
    g = torch.Generator().manual_seed(seed)
    s = torch.randn((T, E), generator=g)
    s[:, torch.randperm(E, generator=g)[:3]] += 2.0      # a few hot experts
    idx = torch.topk(s, k, dim=1).indices.to(torch.int32)
    x = torch.randn((T, 256), generator=g).to(torch.bfloat16)
    return x.cuda(), idx.cuda()


def _outs(T, E, k):
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                slot_of=torch.full((T, k), -7, **i32), row_token=torch.full((T * k,), -7, **i32),
                x_perm=torch.zeros((T * k, 256), dtype=torch.bfloat16, device="cuda"))


def test_noalloc_dispatch_equals_dispatch():
    for n, (T, E, k, e0, e1) in enumerate(CALLS):
        say(f"[gpu] noalloc dispatch call {n}: T={T} E={E} k={k} local=[{e0},{e1})")
        x, idx = _inputs(T, E, k, 100 + n)
        a, b = _outs(T, E, k), _outs(T, E, k)
        nb = L.moe_workspace_bytes(L.WS_DISPATCH, T, 256, E, k, 128)
        assert nb <= L.NOALLOC_SCRATCH_BYTES
        ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device="cuda")
        L.moe_dispatch(x, idx, E, e0, e1, a["counts"], a["offsets"], a["slot_of"],
                       a["row_token"], a["x_perm"], ws)
        L.moe_dispatch_noalloc(x, idx, E, e0, e1, b["counts"], b["offsets"], b["slot_of"],
                               b["row_token"], b["x_perm"])
        torch.cuda.synchronize()
        for name in ("counts", "offsets", "slot_of", "row_token"):
            assert torch.equal(a[name], b[name]), f"call {n}: {name} differs"
        r0, r1 = int(a["offsets"][e0]), int(a["offsets"][e1])
        assert torch.equal(a["x_perm"][r0:r1], b["x_perm"][r0:r1]), f"call {n}: x_perm"
        assert int(a["offsets"][E]) == T * k
        assert torch.equal(a["counts"].long().sum(), torch.tensor(T * k, device="cuda"))
