"""Helpers shared by the GPU parity tests: run the HIP layer, run the oracle on
the same input bytes, compare.

Bars: bit-exact for indices, counts, offsets, the layout map and x_perm;
rel-L2 <= 1e-5 for float32 results (logits, gate weights, the fp32 layer);
rel-L2 <= 1e-2 for bf16 / fp16 / fp8-weight results.  Beside each pooled
rel-L2, every row must also stay within ROW_FACTOR times that bound, so a
few wrong rows cannot hide in a large tensor's pooled norm (a wrong row has a
relative error near 1).  Routing is exact on the GPU's own logits; against
the oracle's own float64 logits, a token may pick differently only where two
experts' scores are within 1e-5 * (|s| + 1) of each other.
"""

import sys

import numpy as np
import torch

from gen.configs import F32, LayerConfig
from gen.inputs import TORCH_DTYPE, make_inputs
from oracle import moe_oracle as O
from oracle.torch_io import stored

TOL_F32 = 1e-5
TOL_16 = 1e-2
ROW_FACTOR = 3.0      # per-row rel-L2 bound = ROW_FACTOR * the pooled bound
NEAR_TIE = 1e-5       # relative score gap below which a top-k flip is a near tie


def tol(cfg: LayerConfig) -> float:
    return TOL_F32 if cfg.act_dtype == F32 else TOL_16


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


def max_row_rel_l2(got, ref) -> float:
    """Largest per-row relative L2 error; a row whose reference is all zero
    must be all zero (its error then counts as 0)."""
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "a row that should be zero is not"
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


def assert_close(got, ref, bound, what):
    """Pooled rel-L2 within bound and every row within ROW_FACTOR * bound."""
    e = rel_l2(got, ref)
    assert e <= bound, f"{what} rel-L2 {e}"
    if len(np.asarray(got)):
        er = max_row_rel_l2(got, ref)
        assert er <= ROW_FACTOR * bound, f"{what}: a row has rel-L2 {er}"
    return e


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def params(cfg: LayerConfig) -> O.LayerParams:
    return O.LayerParams(T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k, I=cfg.I,
                         act_dtype=cfg.act_dtype, w_dtype=cfg.w_dtype, gate=cfg.gate,
                         renorm=cfg.renorm, act=cfg.act, e_begin=cfg.e_begin,
                         e_end=cfg.e_end, inv_temperature=cfg.inv_temperature,
                         min_prob=cfg.min_prob, fp8_dispatch=cfg.fp8_dispatch)


def spec(cfg: LayerConfig):
    from combine_moe_route_02_amd import LayerSpec
    return LayerSpec(T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k, I=cfg.I,
                     act_dtype=TORCH_DTYPE[cfg.act_dtype], gate=cfg.gate,
                     renorm=cfg.renorm, act=cfg.act, e_begin=cfg.e_begin,
                     e_end=cfg.e_end, inv_temperature=cfg.inv_temperature,
                     min_prob=cfg.min_prob, fp8_dispatch=cfg.fp8_dispatch)


def route(cfg: LayerConfig, logits, bias):
    """The oracle's top-k gating with the config's flags, after checking that
    no gate value lies so close to the threshold that float32 rounding could
    decide it (then the kept set is unique and compared bit for bit)."""
    if cfg.min_prob > 0:
        s = O.selection_scores(logits, bias)
        raw = O.raw_gate(s, O.topk_select(s, cfg.k), cfg.gate, cfg.inv_temperature)
        gap = np.abs(raw - cfg.min_prob).min()
        assert gap > 1e-5 * cfg.min_prob, f"a gate value within {gap:.2e} of the threshold"
    return O.route(logits, bias, cfg.k, cfg.gate, cfg.renorm, cfg.inv_temperature,
                   cfg.min_prob)


def gpu_layer(cfg: LayerConfig, inp, fused=False, split=True):
    """Run the whole layer through the C ABI on cuda:0; returns the MoELayer.
    split=False runs the expert GEMMs without a workspace (no k-split)."""
    from combine_moe_route_02_amd import MoELayer
    say(f"[gpu] layer {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} "
        f"{cfg.act_dtype}/{cfg.w_dtype} local=[{cfg.e_begin},{cfg.e_end}) fused={fused} "
        f"split={split}")
    lay = MoELayer(spec(cfg), "cuda", ffn_split=split)
    if inp.get("y_remote") is not None:
        lay.y_perm.copy_(inp["y_remote"])
    if fused:
        lay.forward_fused(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"])
    else:
        lay.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"],
                    inp["w13_scale"], inp["w2_scale"])
    torch.cuda.synchronize()
    return lay


def to_device(inp, device="cuda"):
    return {k: (v.to(device) if v is not None else None) for k, v in inp.items()}


def np_stored(inp):
    return {k: (stored(v) if v is not None else None) for k, v in inp.items()}


def check_routing(cfg, lay, st, check_xperm=True):
    """Integer path, bit-exact, with the oracle run on the GPU's own logits.

    check_xperm=False for the fused kernel, which reads token rows through the
    layout map and writes no permuted copy."""
    logits = lay.logits.cpu().numpy()
    idx, w = route(cfg, logits, st["bias"])
    g_idx = lay.topk_idx.cpu().numpy()
    assert np.array_equal(g_idx, idx), "topk_idx differs"
    assert_close(lay.topk_w.cpu().numpy(), w, TOL_F32, "topk_w")
    counts = O.expert_counts(idx, cfg.E)
    offsets = O.expert_offsets(counts)
    assert np.array_equal(lay.counts.cpu().numpy(), counts)
    assert np.array_equal(lay.offsets.cpu().numpy(), offsets)
    slot_of, row_token = O.layout_map(idx, offsets)
    assert np.array_equal(lay.slot_of.cpu().numpy(), slot_of)
    n_kept = int(offsets[-1])      # rows past the kept picks are not written
    assert np.array_equal(lay.row_token[:n_kept].cpu().numpy(), row_token[:n_kept])
    r0, r1 = int(offsets[cfg.e_begin]), int(offsets[cfg.e_end])
    if check_xperm and cfg.fp8_dispatch:
        # fp8 transport: codes and power-of-two scales are exact, bit for bit
        rows = O.decode(O.gather_rows(st["x"], row_token, r0, r1), cfg.act_dtype)
        codes, scales = O.quantize_rows_e4m3(rows)
        assert np.array_equal(lay.x_q[r0:r1].cpu().numpy(), codes), "x_q differs"
        assert np.array_equal(lay.x_scale[r0:r1].cpu().numpy(), scales), "x_scale differs"
    elif check_xperm:
        xp = stored(lay.x_perm[r0:r1])
        assert np.array_equal(xp, O.gather_rows(st["x"], row_token, r0, r1)), "x_perm differs"
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                slot_of=slot_of, row_token=row_token)


def flipped_tokens(cfg, gpu_logits, own_logits, bias, tokens=None):
    """Tokens whose top-k differs between the oracle's own scores and the GPU's,
    after checking that every such difference is a near tie: wherever the two
    pick lists differ, the two experts' scores (the oracle's own) lie within
    NEAR_TIE * (|s| + 1) of each other.  ``tokens`` selects the rows of
    gpu_logits that own_logits holds (default: all)."""
    g = gpu_logits if tokens is None else gpu_logits[tokens]
    b_ = bias
    a, _ = O.route(g, b_, cfg.k, cfg.gate, cfg.renorm, cfg.inv_temperature, cfg.min_prob)
    b, _ = O.route(own_logits, b_, cfg.k, cfg.gate, cfg.renorm, cfg.inv_temperature,
                   cfg.min_prob)
    flips = np.nonzero((a != b).any(axis=1))[0]
    if len(flips):
        s_own = O.selection_scores(own_logits, bias).astype(np.float64)
        for t in flips:
            for j in range(cfg.k):
                ea, eb = int(a[t, j]), int(b[t, j])
                if ea == eb or ea < 0 or eb < 0:   # -1: the threshold (checked apart)
                    continue
                sa, sb = s_own[t, ea], s_own[t, eb]
                assert abs(sa - sb) <= NEAR_TIE * (abs(sb) + 1.0), (
                    f"token {t}: pick {j} is expert {ea} (GPU) vs {eb} (oracle) with "
                    f"scores {sa!r} / {sb!r}: not a near tie")
    return flips


def full_parity(cfg: LayerConfig, inp_cpu, lay, check_xperm=True):
    """Element-by-element comparison of every output (small layers)."""
    st = np_stored(inp_cpu)
    r = check_routing(cfg, lay, st, check_xperm)
    p = params(cfg)
    own = O.router_logits(O.decode(st["x"], cfg.act_dtype),
                          O.decode(st["w_router"], cfg.act_dtype))
    assert rel_l2(r["logits"], own) <= TOL_F32
    flips = flipped_tokens(cfg, r["logits"], own, st["bias"])
    assert len(flips) <= max(1, cfg.T // 1000), f"top-k flips at {flips[:10]}"
    ref = O.layer_forward(p, st["x"], st["w_router"], st["bias"], st["w13"], st["w2"],
                          st["w13_scale"], st["w2_scale"], st["y_remote"],
                          logits=r["logits"])
    r0, r1 = int(r["offsets"][cfg.e_begin]), int(r["offsets"][cfg.e_end])
    y = O.decode(stored(lay.y_perm), cfg.act_dtype)
    if r1 > r0:
        assert_close(y[r0:r1], ref["y_perm"][r0:r1], tol(cfg), "y_perm")
    out = O.decode(stored(lay.out), cfg.act_dtype)
    e_o = assert_close(out, ref["out"], tol(cfg), "out")
    return dict(out_rel=e_o, flips=len(flips))
