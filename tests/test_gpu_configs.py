"""GPU parity on the five layer shapes at full size, in the launch
configuration the benchmark times.

The integer path (indices, counts, offsets, layout map, the permute-gather)
is compared bit for bit over every token, with the oracle re-run on the
GPU's logits.  The router logits of every token are compared with the
oracle's own float64 logits, and every token whose top-k would differ under
the oracle's own scores must be a near tie.  The rest of floating point is
compared on samples the oracle computes one by one: expert outputs at
sampled rows (including the first and last row of every local expert's
segment) and the combined output of sampled tokens, pooled and per row.
"""

import numpy as np
import pytest
import torch

from gen.configs import CONFIGS
from gen.inputs import make_inputs
from oracle import moe_oracle as O
from oracle.torch_io import stored
from tests.harness import TOL_F32, assert_close, check_routing, flipped_tokens, \
    full_parity, gpu_layer, params, rel_l2, say, tol

pytestmark = pytest.mark.gpu


def test_c1_full():
    cfg = CONFIGS["c1"]
    inp = make_inputs(cfg, "cpu")
    lay = gpu_layer(cfg, {k: (v.cuda() if v is not None else None) for k, v in inp.items()})
    res = full_parity(cfg, inp, lay)
    say(f"  c1 out rel-L2 {res['out_rel']:.3e}")


def sampled_parity(cfg, inp, lay, n_tokens=48, seed=7, check_xperm=True):
    """Bit-exact integer path over all tokens; float outputs on samples."""
    st = {"x": stored(inp["x"]), "w_router": stored(inp["w_router"]),
          "bias": stored(inp["bias"]) if inp["bias"] is not None else None}
    r = check_routing(cfg, lay, st, check_xperm)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))

    # router logits of every token against the oracle's own, in chunks; a
    # top-k that would differ under the oracle's scores must be a near tie
    wr64 = O.decode(st["w_router"], cfg.act_dtype)
    num = den = 0.0
    n_flips = 0
    for c0 in range(0, cfg.T, 4096):
        c1 = min(cfg.T, c0 + 4096)
        own = O.router_logits(O.decode(st["x"][c0:c1], cfg.act_dtype), wr64)
        num += float(np.sum((r["logits"][c0:c1].astype(np.float64) - own) ** 2))
        den += float(np.sum(own ** 2))
        n_flips += len(flipped_tokens(cfg, r["logits"], own, st["bias"],
                                      tokens=np.arange(c0, c1)))
    e_l = (num / den) ** 0.5
    say(f"  {cfg.name}: logits rel-L2 {e_l:.3e} over all {cfg.T} tokens, "
        f"{n_flips} near-tie top-k flips")
    assert e_l <= TOL_F32, f"logits rel-L2 {e_l}"

    # rows to check: the sampled tokens' picks + each local segment's ends
    off, slot_of, idx = r["offsets"], r["slot_of"], r["idx"]
    rows = set(r_ for r_ in slot_of[toks].ravel().tolist() if r_ >= 0)   # -1: dropped
    for e in range(cfg.e_begin, cfg.e_end):
        if off[e + 1] > off[e]:
            rows.update([int(off[e]), int(off[e + 1]) - 1])
    rows = np.array(sorted(rows), dtype=np.int64)
    y_gpu = O.decode(stored(lay.y_perm[torch.as_tensor(rows, device="cuda")]), cfg.act_dtype)
    y_ref = np.empty_like(y_gpu)
    expert_of_row = np.searchsorted(off, rows, side="right") - 1
    remote = None
    if inp["y_remote"] is not None:
        remote = O.decode(stored(inp["y_remote"][torch.as_tensor(rows, device=inp["y_remote"].device)]),
                          cfg.act_dtype)
    p = params(cfg)
    local_sel = (expert_of_row >= cfg.e_begin) & (expert_of_row < cfg.e_end)
    if remote is not None:
        y_ref[~local_sel] = remote[~local_sel]
    for e in np.unique(expert_of_row[local_sel]):
        sel = np.nonzero(expert_of_row == e)[0]
        el = int(e) - cfg.e_begin
        w13 = stored(inp["w13"][el])
        w2 = stored(inp["w2"][el])
        s13 = stored(inp["w13_scale"][el])[None] if inp["w13_scale"] is not None else None
        s2 = stored(inp["w2_scale"][el])[None] if inp["w2_scale"] is not None else None
        W13, W2 = O.expert_weights(p, w13[None], w2[None], s13, s2, 0)
        X = O.decode(st["x"][r["row_token"][rows[sel]]], cfg.act_dtype)
        if cfg.fp8_dispatch:      # the FFN sees the dequantised fp8 rows
            codes, sc = O.quantize_rows_e4m3(X)
            X = O.e4m3_decode(codes) * sc.astype(np.float64)[:, None]
        y_ref[sel] = O.expert_ffn(X, W13, W2, cfg.act, cfg.act_dtype)
    loc = np.nonzero(local_sel)[0]
    if len(loc):
        e_y = assert_close(y_gpu[loc], y_ref[loc], tol(cfg), "y_perm")
        say(f"  {cfg.name}: y_perm rel-L2 {e_y:.3e} over {len(loc)} rows")
    if remote is not None and (~local_sel).any():
        assert np.array_equal(y_gpu[~local_sel], remote[~local_sel])

    # combine of sampled tokens, from the oracle's rows
    pos = {int(rw): i for i, rw in enumerate(rows)}
    slot_c = np.vectorize(lambda r_: pos.get(r_, -1))(slot_of[toks]).astype(np.int64)
    out_ref = O.combine(y_ref, slot_c, r["w"][toks], cfg.act_dtype,
                        tokens=np.arange(len(toks)))
    out_gpu = O.decode(stored(lay.out[torch.as_tensor(toks, device="cuda")]), cfg.act_dtype)
    e_o = assert_close(out_gpu, out_ref, tol(cfg), "out")
    say(f"  {cfg.name}: out rel-L2 {e_o:.3e} over {len(toks)} tokens")
    return r


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_full_size_config(name):
    cfg = CONFIGS[name]
    say(f"[gen] {name} on cuda")
    inp = make_inputs(cfg, "cuda")
    lay = gpu_layer(cfg, inp)
    r = sampled_parity(cfg, inp, lay)
    counts = r["counts"].astype(np.float64)
    if name == "c4":
        ratio = counts.max() / counts.mean()
        say(f"  c4 load max/mean {ratio:.2f}, local rows "
            f"{int(r['offsets'][cfg.e_end] - r['offsets'][cfg.e_begin])}")
        assert abs(ratio - 10.0) < 0.5


def test_c5_fp8_dispatch():
    """The decode layer with its dispatched rows sent as E4M3 (fp8 x fp8 GEMM-1):
    codes and scales bit-exact, outputs against the oracle's fp8 transport."""
    cfg = CONFIGS["c5"].with_(fp8_dispatch=True)
    say("[gen] c5 (fp8 dispatch) on cuda")
    inp = make_inputs(cfg, "cuda")
    lay = gpu_layer(cfg, inp)
    sampled_parity(cfg, inp, lay, n_tokens=64)
