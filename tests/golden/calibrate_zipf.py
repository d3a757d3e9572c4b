"""Find the log-Zipf bias strength of the 256-expert layer (c4) with the oracle.

The workload asks for Zipf(1.2) expert popularity with the hot expert at
about ten times the mean load.  The generator adds a selection bias
-1.2 * alpha * ln(rank_e); this script bisects alpha so that, on this seed's
draw, the busiest expert receives 10x the mean load over all 256 experts
when routing is done by the oracle, and writes the result to c4_zipf.json.

Run:  python tests/golden/calibrate_zipf.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gen.configs import CONFIGS  # noqa: E402
from gen.inputs import make_inputs, zipf_bias  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from oracle.torch_io import stored  # noqa: E402

TARGET = 10.0


def load_ratio(cfg, logits, alpha):
    bias = stored(zipf_bias(cfg.with_(zipf_alpha=alpha)))
    idx, _ = O.route(logits, bias, cfg.k, cfg.gate, cfg.renorm)
    counts = O.expert_counts(idx, cfg.E).astype(np.float64)
    return counts.max() / counts.mean(), counts


def main():
    cfg = CONFIGS["c4"]
    inp = make_inputs(cfg, "cpu", with_weights=False)
    x = O.decode(stored(inp["x"]), cfg.act_dtype)
    wr = O.decode(stored(inp["w_router"]), cfg.act_dtype)
    logits = O.router_logits(x, wr)
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        r, _ = load_ratio(cfg, logits, mid)
        if r < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(hi, 4)
    ratio, counts = load_ratio(cfg, logits, alpha)
    loc = counts[cfg.e_begin:cfg.e_end]
    res = {
        "source": "workload: Zipf(1.2) expert popularity with the hot expert at "
                  "about 10x the mean load; alpha found by bisection with the "
                  "oracle's routing on seed %d" % cfg.seed,
        "alpha": alpha,
        "max_over_mean": ratio,
        "local_rows": int(loc.sum()),
        "local_min": int(loc.min()),
        "local_max": int(loc.max()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c4_zipf.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=2)
    print(json.dumps(res, indent=2))


if __name__ == "__main__":
    main()
