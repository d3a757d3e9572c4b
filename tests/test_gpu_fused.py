"""The fused dispatch -> GEMM-1 -> GEMM-2 -> combine kernel against the
unfused path without the k-split workspace (same tiles and accumulation
order: bit-identical results) and against the oracle at full size."""

import pytest
import torch

from gen.configs import CONFIGS
from gen.inputs import make_inputs
from tests.harness import full_parity, gpu_layer, say, to_device
from tests.test_gpu_configs import sampled_parity
from tests.test_gpu_small import GRID, small

pytestmark = pytest.mark.gpu

FUSED_SMALL = [c for c in GRID if c.act_dtype != "f32" and c.w_dtype == c.act_dtype
               and c.act == "swiglu"]
FUSED_SMALL.append(small("fused_hot", 700, 256, 8, 2, 128, bias="normal", seed_off=40))


def _fused_ws_ok(lay):
    assert lay.fused_status() == 0, "fused kernel reported a wait timeout"


def _compare(cfg, a, b):
    r0 = int(a.offsets[cfg.e_begin])
    r1 = int(a.offsets[cfg.e_end])
    for n in ["topk_idx", "counts", "offsets", "slot_of"]:
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    n_kept = int(a.offsets[-1])    # row_token past the kept picks is not written
    assert torch.equal(a.row_token[:n_kept], b.row_token[:n_kept])
    assert torch.equal(a.out, b.out), "out differs from the unfused path"
    assert torch.equal(a.y_perm[r0:r1], b.y_perm[r0:r1])
    assert torch.equal(a.h[: r1 - r0], b.h[: r1 - r0])


@pytest.mark.parametrize("cfg", FUSED_SMALL, ids=[c.name for c in FUSED_SMALL])
def test_fused_equals_unfused_small(cfg):
    inp = make_inputs(cfg, "cpu")
    dev = to_device(inp)
    if cfg.name == "fused_hot":
        dev["bias"] = torch.zeros(8, device="cuda")
        dev["bias"][5] = 3.0       # one expert takes most of the load
    a = gpu_layer(cfg, dev, fused=True)
    _fused_ws_ok(a)
    b = gpu_layer(cfg, dev, fused=False, split=False)
    _compare(cfg, a, b)
    if cfg.name != "fused_hot":
        full_parity(cfg, inp, a, check_xperm=False)
    # a second call on the same workspace: the first left its counters at zero
    first = a.out.clone()
    a.out.zero_()
    a.fused(dev["x"], dev["w13"], dev["w2"])
    torch.cuda.synchronize()
    _fused_ws_ok(a)
    assert torch.equal(a.out, first), "second fused call differs"


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_fused_full_size(name):
    cfg = CONFIGS[name]
    say(f"[gen] {name} on cuda")
    inp = make_inputs(cfg, "cuda")
    a = gpu_layer(cfg, inp, fused=True)
    _fused_ws_ok(a)
    b = gpu_layer(cfg, inp, fused=False, split=False)
    _compare(cfg, a, b)
    if name == "c4":
        sampled_parity(cfg, inp, a, n_tokens=24, check_xperm=False)
