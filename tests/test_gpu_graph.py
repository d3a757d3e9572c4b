"""The decode layer (fp8 experts) captured once in a hipGraph and replayed.

The whole layer (router, top-k, dispatch, expert FFN, combine) is captured
on the graph's stream; replays on two different token batches give two
different routings, and each replay is checked against the oracle (the
per-expert counts are read on the device, never by the host).  Inputs are
refreshed with plain copies outside the graph, and each replay is compared
with an eager run of the same batch.
"""

import numpy as np
import pytest
import torch

from gen.configs import CONFIGS, STREAM_X
from gen.inputs import make_inputs, normal
from tests.harness import say, spec
from tests.test_gpu_configs import sampled_parity

pytestmark = pytest.mark.gpu


def test_decode_layer_graph_replay():
    from combine_moe_route_02_amd import MoELayer
    cfg = CONFIGS["c5"]
    inp = make_inputs(cfg, "cuda")
    lay = MoELayer(spec(cfg), "cuda")
    x_static = inp["x"].clone()
    args = (inp["w_router"], inp["bias"], inp["w13"], inp["w2"], inp["w13_scale"],
            inp["w2_scale"])

    def fwd():
        lay.forward(x_static, *args)

    # warm up on a side stream, then capture on the graph's stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.y_perm.copy_(inp["y_remote"])
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("[gpu] capturing the decode layer")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()

    counts_seen = []
    for trial in range(2):
        xb = normal((cfg.T, cfg.H), inp["x"].dtype, cfg.seed + 1000 + trial, STREAM_X, 1.0,
                    "cuda")
        x_static.copy_(xb)
        lay.y_perm.copy_(inp["y_remote"])
        torch.cuda.synchronize()
        say(f"[gpu] replay {trial}")
        g.replay()
        torch.cuda.synchronize()
        got = {n: getattr(lay, n).clone() for n in ["topk_idx", "offsets", "out"]}
        counts_seen.append(lay.counts.cpu().numpy().copy())
        # the replay equals an eager run of the same batch
        lay.y_perm.copy_(inp["y_remote"])
        fwd()
        torch.cuda.synchronize()
        for n, v in got.items():
            assert torch.equal(v, getattr(lay, n)), n
        # and the oracle on this batch
        g.replay()
        torch.cuda.synchronize()
        trial_inp = dict(inp)
        trial_inp["x"] = x_static
        sampled_parity(cfg, trial_inp, lay, n_tokens=16, seed=trial)
    assert not np.array_equal(counts_seen[0], counts_seen[1]), \
        "the two batches should route differently"
