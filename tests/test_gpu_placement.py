"""Placement of replicated experts and the online load statistics against
the oracle, and a layer whose hot experts are replicated (the copies hold
their expert's weights): the same output as the unreplicated layer, bit for
bit, since every row meets the same weights in the same k order."""

import dataclasses

import numpy as np
import pytest
import torch

from gen.inputs import make_inputs
from oracle import moe_oracle as O
from oracle.torch_io import stored
from tests.harness import gpu_layer, np_stored, params, rel_l2, say, spec, to_device, tol
from tests.test_gpu_small import small

pytestmark = pytest.mark.gpu


def test_place_and_stats_match_oracle():
    from combine_moe_route_02_amd import moe_expert_load_stats, moe_place_experts
    r = np.random.default_rng(90)
    T, E, k = 3000, 64, 6
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[r.random((T, k)) < 0.1] = -1
    ncopy = r.integers(1, 4, size=E)
    rep_off = np.concatenate([[0], np.cumsum(ncopy)]).astype(np.int32)
    rep_phys = r.permutation(int(ncopy.sum())).astype(np.int32)
    E_phys = int(ncopy.sum())
    say(f"[gpu] place T={T} E={E} k={k} E_phys={E_phys}")
    d_idx = torch.from_numpy(idx).cuda()
    out = torch.empty_like(d_idx)
    moe_place_experts(d_idx, E, E_phys, torch.from_numpy(rep_off).cuda(),
                      torch.from_numpy(rep_phys).cuda(), out)
    stats = torch.zeros(E, dtype=torch.int64, device="cuda")
    for _ in range(3):
        moe_expert_load_stats(d_idx, E, stats)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.place_experts(idx, rep_off, rep_phys))
    assert np.array_equal(stats.cpu().numpy().astype(np.uint64), 3 * O.expert_load(idx, E))


def test_replicated_hot_experts_give_the_same_layer():
    from combine_moe_route_02_amd import MoELayer
    cfg = small("placed", 700, 256, 8, 2, 128, bias="normal", seed_off=70)
    inp = make_inputs(cfg, "cpu")
    bias = torch.zeros(8)
    bias[3], bias[5] = 2.0, 1.0            # two hot experts
    inp["bias"] = bias
    dev = to_device(inp)
    base = gpu_layer(cfg, dev, split=False)

    ncopy = np.array([1, 1, 1, 3, 1, 2, 1, 1])
    rep_off = np.concatenate([[0], np.cumsum(ncopy)]).astype(np.int32)
    rep_phys = np.random.default_rng(71).permutation(11).astype(np.int32)
    owner = np.empty(11, np.int64)
    for e in range(8):
        owner[rep_phys[rep_off[e]:rep_off[e + 1]]] = e
    own = torch.from_numpy(owner).cuda()
    w13, w2 = dev["w13"][own].contiguous(), dev["w2"][own].contiguous()
    say("[gpu] layer with 3 copies of expert 3 and 2 of expert 5 (11 physical slots)")
    lay = MoELayer(dataclasses.replace(spec(cfg), E_phys=11, e_end=11), "cuda",
                   ffn_split=False)
    lay.set_placement(torch.from_numpy(rep_off).cuda(), torch.from_numpy(rep_phys).cuda())
    lay.enable_load_stats()
    lay.forward(dev["x"], dev["w_router"], dev["bias"], w13, w2)
    torch.cuda.synchronize()

    assert torch.equal(lay.topk_idx, base.topk_idx)
    assert np.array_equal(lay.load_stats.cpu().numpy(), base.counts.cpu().numpy())
    counts = lay.counts.cpu().numpy()
    for e in (3, 5):                        # the hot experts' rows are spread
        assert counts[rep_phys[rep_off[e]:rep_off[e + 1]]].min() > 0
    d = rel_l2(O.decode(stored(lay.out), cfg.act_dtype), O.decode(stored(base.out), cfg.act_dtype))
    assert torch.equal(lay.out, base.out), f"out differs from the unreplicated layer ({d:.2e})"

    # the placed layer against the oracle on the GPU's own scores
    st = np_stored(inp)
    p = dataclasses.replace(params(cfg), e_end=11)
    ref = O.layer_forward(p, st["x"], st["w_router"], st["bias"], st["w13"][owner],
                          st["w2"][owner], logits=lay.logits.cpu().numpy(),
                          placement=(rep_off, rep_phys, 11))
    assert np.array_equal(lay.topk_phys.cpu().numpy(), ref["topk_phys"])
    assert np.array_equal(counts, ref["counts"])
    assert np.array_equal(lay.offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(lay.slot_of.cpu().numpy(), ref["slot_of"])
    e_o = rel_l2(O.decode(stored(lay.out), cfg.act_dtype), ref["out"])
    say(f"  placed layer: out rel-L2 {e_o:.3e}")
    assert e_o <= tol(cfg)
