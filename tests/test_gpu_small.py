"""GPU parity on small shapes: every output element against the oracle.

The shapes span several MFMA tiles with ragged tails, and the edge cases of
the method: one expert, k = E, all tokens on one expert, empty experts, no
local expert, a single token, no tokens, mass ties in the scores, and every
router projection kernel (staged MFMA tiles for many experts and large
batches, per-lane-loaded 16x16 MFMA tiles otherwise, the vector kernel for
float32 and for rows that are not a multiple of 32).
"""

import numpy as np
import pytest
import torch

from gen.configs import BASE_SEED, BF16, F16, F32, FP8_E4M3, GELU, SIGMOID, SOFTMAX, \
    SWIGLU, LayerConfig
from gen.inputs import make_inputs
from oracle import moe_oracle as O
from oracle.torch_io import stored
from tests.harness import TOL_F32, check_routing, full_parity, gpu_layer, np_stored, \
    params, rel_l2, route, say, spec, to_device

pytestmark = pytest.mark.gpu


def small(name, T, H, E, k, I, act_dtype=BF16, w_dtype=None, gate=SOFTMAX, renorm=False,
          act=SWIGLU, e_begin=0, e_end=None, bias=None, remote=False, seed_off=0,
          inv_t=1.0, min_prob=0.0, fp8d=False):
    return LayerConfig(name, T=T, H=H, E=E, k=k, I=I, act_dtype=act_dtype,
                       w_dtype=w_dtype or act_dtype, gate=gate, renorm=renorm, act=act,
                       e_begin=e_begin, e_end=E if e_end is None else e_end,
                       seed=BASE_SEED + 100 + seed_off, bias=bias, remote_rows=remote,
                       inv_temperature=inv_t, min_prob=min_prob, fp8_dispatch=fp8d)


GRID = [
    small("bf16_tiles", 1000, 512, 8, 2, 256, renorm=True, bias="normal", seed_off=1),
    small("f16_e16", 777, 256, 16, 4, 128, act_dtype=F16, seed_off=2),
    small("bf16_ep_share", 300, 256, 64, 6, 128, gate=SIGMOID, e_begin=8, e_end=40,
          remote=True, seed_off=3),
    small("f32_gelu", 255, 128, 8, 2, 256, act_dtype=F32, act=GELU, seed_off=4),
    small("fp8_ep_share", 64, 256, 256, 8, 128, w_dtype=FP8_E4M3, gate=SIGMOID,
          e_begin=0, e_end=32, remote=True, seed_off=5),
    small("bf16_router_mfma", 1100, 256, 256, 8, 128, gate=SIGMOID, seed_off=6),
    small("bf16_router_valu_e256", 129, 256, 256, 8, 128, gate=SIGMOID, seed_off=16),
    small("router_valu_e200", 70, 256, 200, 4, 128, seed_off=17),
    small("dense_e1", 100, 256, 1, 1, 128, renorm=True, seed_off=7),
    small("k_equals_e", 50, 256, 4, 4, 128, seed_off=8),
    small("one_token", 1, 256, 8, 2, 128, seed_off=9),
    small("bf16_gelu", 200, 256, 8, 2, 256, act=GELU, seed_off=10),
    small("no_local_expert", 90, 256, 8, 2, 128, e_begin=4, e_end=4, remote=True,
          seed_off=11),
    small("f16_e64_k1", 513, 256, 64, 1, 128, act_dtype=F16, seed_off=12),
    # fp8 weights: decode tile (few rows per expert, some experts over one
    # 32-row tile), GELU, and the many-rows fp8 path
    small("fp8_multi_mtile", 96, 256, 8, 2, 256, w_dtype=FP8_E4M3, seed_off=13),
    small("fp8_gelu", 80, 256, 8, 2, 256, w_dtype=FP8_E4M3, act=GELU, seed_off=14),
    small("fp8_large_m", 400, 256, 8, 2, 256, w_dtype=FP8_E4M3, seed_off=15),
    # the one-launch layout for few experts: 17-32 experts, and the largest
    # batch it takes (32768 picks)
    small("bf16_e32", 600, 256, 32, 4, 128, gate=SIGMOID, seed_off=19),
    small("f16_e24", 520, 256, 24, 3, 128, act_dtype=F16, seed_off=20),
    small("bf16_e32_max_picks", 4096, 256, 32, 8, 128, gate=SIGMOID, seed_off=21),
    # long K: the GEMMs' sparse last round is split over K (parts of 4+ k-steps)
    small("bf16_ksplit", 300, 2048, 8, 2, 1024, seed_off=18),
    # gating variants: temperature, and the minimum-probability threshold
    # (dropped picks: index -1, no row, nothing to combine); the page's
    # temperature 0.3 with threshold 0.05, renormalised survivors, sigmoid on
    # an expert-parallel share, fp32, fp8 weights, and a threshold above
    # every gate value (all picks dropped: empty FFN, zero output)
    small("bf16_tau03", 400, 256, 16, 4, 128, inv_t=1 / 0.3, seed_off=50),
    small("bf16_tau2", 400, 256, 16, 4, 128, inv_t=0.5, seed_off=51),
    small("bf16_threshold", 500, 256, 16, 4, 128, inv_t=1 / 0.3, min_prob=0.05,
          seed_off=52),
    small("f16_threshold_renorm", 300, 256, 8, 2, 256, act_dtype=F16, renorm=True,
          min_prob=0.3, seed_off=53),
    small("sigmoid_threshold_ep", 200, 256, 64, 6, 128, gate=SIGMOID, e_begin=8,
          e_end=40, remote=True, min_prob=0.83, seed_off=54),
    small("f32_threshold", 255, 128, 8, 2, 256, act_dtype=F32, act=GELU, min_prob=0.2,
          seed_off=55),
    small("fp8_threshold", 64, 256, 256, 8, 128, w_dtype=FP8_E4M3, gate=SIGMOID,
          e_end=32, remote=True, min_prob=0.89, seed_off=56),
    small("all_dropped", 100, 256, 8, 2, 128, min_prob=1.0, seed_off=57),
    # fp8 dispatch transport: E4M3 rows with a power-of-two scale per row into
    # the fp8 x fp8 GEMM-1 (decode batch on an EP share, GELU, many rows per
    # expert, dropped picks)
    small("fp8d_ep_share", 64, 256, 256, 8, 128, w_dtype=FP8_E4M3, gate=SIGMOID,
          e_end=32, remote=True, fp8d=True, seed_off=60),
    small("fp8d_gelu", 80, 256, 8, 2, 256, w_dtype=FP8_E4M3, act=GELU, fp8d=True,
          seed_off=61),
    small("fp8d_many_rows", 400, 512, 8, 2, 256, w_dtype=FP8_E4M3, fp8d=True,
          seed_off=62),
    small("fp8d_threshold", 64, 256, 256, 8, 128, w_dtype=FP8_E4M3, gate=SIGMOID,
          e_end=32, remote=True, min_prob=0.89, fp8d=True, seed_off=56),
]


# Router projection alone, at the edges of each kernel's tiling: partial token
# tiles, padded expert tiles, fewer 32-wide k steps than waves, a one-token
# last tile of the staged kernel, several expert tiles, and 16-bit rows that
# are not a multiple of 32 (the vector kernel).
ROUTER_SHAPES = [
    small("r_mfma16_e8_h96", 33, 96, 8, 2, 64, seed_off=70),
    small("r_mfma16_e40_f16", 47, 512, 40, 3, 64, act_dtype=F16, seed_off=71),
    small("r_mfma16_e256_t1", 1, 1024, 256, 8, 64, gate=SIGMOID, seed_off=72),
    small("r_valu_h200", 20, 200, 8, 2, 64, seed_off=73),
    small("r_staged_e256_t1025", 1025, 128, 256, 8, 64, gate=SIGMOID, seed_off=74),
    small("r_staged_e512_f16", 1090, 256, 512, 4, 64, act_dtype=F16, seed_off=75),
    # E a multiple of 128 but not 256: three 128-expert tiles per token tile
    small("r_gemm_e384_t1030", 1030, 256, 384, 8, 64, gate=SIGMOID, seed_off=76),
    # one expert tile per token tile; a single k-step, and two
    small("r_pair_e128_h64", 1100, 64, 128, 4, 64, seed_off=77),
    small("r_pair_e256_h128_t2049", 2049, 128, 256, 8, 64, gate=SIGMOID, seed_off=78),
]


@pytest.mark.parametrize("cfg", ROUTER_SHAPES, ids=[c.name for c in ROUTER_SHAPES])
def test_router_projection_paths(cfg):
    from combine_moe_route_02_amd import MoELayer
    inp = make_inputs(cfg, "cpu", with_weights=False)
    st = np_stored(inp)
    say(f"[gpu] route {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    lay = MoELayer(spec(cfg), "cuda")
    dev = to_device(inp)
    lay.route(dev["x"], dev["w_router"], dev["bias"])
    torch.cuda.synchronize()
    logits = lay.logits.cpu().numpy()
    own = O.router_logits(O.decode(st["x"], cfg.act_dtype),
                          O.decode(st["w_router"], cfg.act_dtype))
    assert rel_l2(logits, own) <= TOL_F32
    idx, w = route(cfg, logits, st["bias"])
    assert np.array_equal(lay.topk_idx.cpu().numpy(), idx)
    assert rel_l2(lay.topk_w.cpu().numpy(), w) <= TOL_F32


def test_router_logits_off_alignment():
    """Logits written to a buffer 4 bytes off 16-byte alignment (the
    projection stores single floats, so any 4-byte alignment serves): the
    same logits, bit for bit, and the same top-k."""
    from combine_moe_route_02_amd import MoELayer, _lib as L
    cfg = ROUTER_SHAPES[-1]
    inp = to_device(make_inputs(cfg, "cpu", with_weights=False))
    say(f"[gpu] route off alignment {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E}")
    lay = MoELayer(spec(cfg), "cuda")
    lay.route(inp["x"], inp["w_router"], inp["bias"])
    buf = torch.empty(cfg.T * cfg.E + 4, dtype=torch.float32, device="cuda")
    odd = buf[1:1 + cfg.T * cfg.E].view(cfg.T, cfg.E)
    assert odd.data_ptr() % 16 != 0
    idx = torch.empty_like(lay.topk_idx)
    w = torch.empty_like(lay.topk_w)
    s = lay.spec
    from combine_moe_route_02_amd.layer import GATES
    L.moe_route(inp["x"], inp["w_router"], inp["bias"], s.k, GATES[s.gate], s.renorm,
                s.inv_temperature, odd, idx, w, min_prob=s.min_prob)
    torch.cuda.synchronize()
    assert torch.equal(odd, lay.logits)
    assert torch.equal(idx, lay.topk_idx) and torch.equal(w, lay.topk_w)


@pytest.mark.parametrize("cfg", GRID, ids=[c.name for c in GRID])
def test_small_layer_parity(cfg):
    inp = make_inputs(cfg, "cpu")
    lay = gpu_layer(cfg, to_device(inp))
    res = full_parity(cfg, inp, lay)
    say(f"  {cfg.name}: out rel-L2 {res['out_rel']:.3e}, flips {res['flips']}")


def test_all_tokens_on_one_expert():
    cfg = small("hot_expert", 600, 256, 8, 1, 128, seed_off=20)
    inp = make_inputs(cfg, "cpu")
    bias = torch.zeros(8, dtype=torch.float32)
    bias[3] = 100.0
    inp["bias"] = bias
    lay = gpu_layer(cfg.with_(bias="normal"), to_device(inp))
    counts = lay.counts.cpu().numpy()
    assert counts.tolist() == [0, 0, 0, 600, 0, 0, 0, 0]
    full_parity(cfg.with_(bias="normal"), inp, lay)


def test_empty_input():
    cfg = small("empty", 0, 256, 8, 2, 128, seed_off=21)
    inp = make_inputs(cfg, "cpu")
    lay = gpu_layer(cfg, to_device(inp))
    assert lay.counts.cpu().tolist() == [0] * 8
    assert lay.offsets.cpu().tolist() == [0] * 9


@pytest.mark.parametrize("T", [500, 4100])
def test_mass_ties_in_scores(T):
    """Scores in {-1, -0, +0, 1}: selection must follow (score desc, index asc).
    500 tokens take the wave-per-token selection, 4100 the 16-lane one
    (E <= 256)."""
    from combine_moe_route_02_amd import MoELayer
    for E, k in [(16, 4), (256, 8), (8, 8), (1024, 32)]:
        cfg = small(f"ties_{E}", T, 256, E, k, 128, seed_off=30 + E)
        lay = MoELayer(spec(cfg), "cuda")
        g = torch.Generator().manual_seed(E)
        s = torch.randint(-1, 2, (T, E), generator=g).float()
        s[torch.rand((T, E), generator=g) < 0.2] = -0.0
        say(f"[gpu] route ties T={T} E={E} k={k}")
        lay.logits.copy_(s.cuda())
        lay.route_from_logits()
        torch.cuda.synchronize()
        idx, w = O.route(s.numpy(), None, k, "softmax", False)
        assert np.array_equal(lay.topk_idx.cpu().numpy(), idx)
        assert rel_l2(lay.topk_w.cpu().numpy(), w) <= TOL_F32


# (gate, renorm, inverse temperature, threshold) on the same scores
GATE_CASES = [("softmax", False, 1 / 0.3, 0.0), ("softmax", True, 1.0, 0.0),
              ("sigmoid", True, 1.0, 0.0), ("softmax", False, 0.0, 0.0),
              ("softmax", False, 1 / 0.3, 0.05), ("softmax", True, 1.0, 0.04),
              ("sigmoid", True, 1.0, 0.93), ("sigmoid", False, 1.0, 0.985)]


@pytest.mark.parametrize("T", [300, 600])
def test_gate_variants_on_given_scores(T):
    """Temperature, sigmoid and renormalisation on the same scores (300
    tokens: wave-per-token selection; 600, the same 300 rows twice: the
    16-lane one).  The scores keep every gate value well away from the
    thresholds, so the kept sets are unique."""
    from combine_moe_route_02_amd import MoELayer
    g = torch.Generator().manual_seed(5)
    s = torch.randn((300, 64), generator=g) * 2
    bias = torch.randn(64, generator=g)
    s = s.repeat(T // 300, 1)
    for gate, renorm, invt, thr in GATE_CASES:
        cfg = small("gates", T, 256, 64, 6, 128, gate=gate, renorm=renorm,
                    inv_t=invt, min_prob=thr)
        lay = MoELayer(spec(cfg), "cuda")
        lay.logits.copy_(s.cuda())
        say(f"[gpu] route T={T} gate={gate} renorm={renorm} inv_t={invt} min_prob={thr}")
        lay.route_from_logits(bias.cuda())
        torch.cuda.synchronize()
        idx, w = route(cfg, s.numpy(), bias.numpy())
        assert np.array_equal(lay.topk_idx.cpu().numpy(), idx)
        assert rel_l2(lay.topk_w.cpu().numpy(), w) <= TOL_F32


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (128, 8), (256, 8), (256, 16)])
def test_topk_paths_agree_bitwise(E, k):
    """The 16-lane selection (large batches) and the wave-per-token one
    (small batches) return the same picks and the same weight bits for the
    same scores, so a token's routing does not depend on its batch size."""
    from combine_moe_route_02_amd import MoELayer
    T_big, T_small = 4100, 500
    g = torch.Generator().manual_seed(E + k)
    s = torch.randn((T_big, E), generator=g) * 2
    bias = torch.randn(E, generator=g)
    for gate, renorm, invt, thr in GATE_CASES:
        out = []
        for T in (T_big, T_small):
            cfg = small("paths", T, 256, E, k, 128, gate=gate, renorm=renorm,
                        inv_t=invt, min_prob=thr)
            lay = MoELayer(spec(cfg), "cuda")
            lay.logits.copy_(s[:T].cuda())
            say(f"[gpu] route paths T={T} E={E} k={k} gate={gate} renorm={renorm}")
            lay.route_from_logits(bias.cuda())
            torch.cuda.synchronize()
            out.append((lay.topk_idx.cpu(), lay.topk_w.cpu()))
        assert torch.equal(out[0][0][:T_small], out[1][0])
        assert torch.equal(out[0][1][:T_small], out[1][1])


def test_repeat_runs_are_bitwise_identical():
    cfg = GRID[0]
    inp = to_device(make_inputs(cfg, "cpu"))
    a = gpu_layer(cfg, inp)
    b = gpu_layer(cfg, inp)
    for name in ["logits", "topk_idx", "topk_w", "counts", "offsets", "slot_of",
                 "row_token", "y_perm", "out"]:
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    r1 = int(a.offsets[cfg.e_end])           # rows written by dispatch and the FFN
    assert torch.equal(a.x_perm[:r1], b.x_perm[:r1])
    assert torch.equal(a.h[:r1], b.h[:r1])


def test_ksplit_matches_unsplit():
    """The k-split of the last round changes only the fp32 summation order."""
    cfg = small("ksplit_cmp", 300, 2048, 8, 2, 1024, seed_off=19)
    inp = make_inputs(cfg, "cpu")
    dev = to_device(inp)
    a = gpu_layer(cfg, dev, split=True)
    b = gpu_layer(cfg, dev, split=False)
    r0, r1 = int(a.offsets[cfg.e_begin]), int(a.offsets[cfg.e_end])
    ya = O.decode(stored(a.y_perm[r0:r1]), cfg.act_dtype)
    yb = O.decode(stored(b.y_perm[r0:r1]), cfg.act_dtype)
    e = rel_l2(ya, yb)
    say(f"  split vs unsplit y_perm rel-L2 {e:.3e}")
    assert e <= 1e-3
    full_parity(cfg, inp, a)


def test_fp8_dispatch_accuracy_against_the_16bit_transport():
    """The fp8 transport changes the layer's output by the rounding of E4M3
    activations: the GPU's change (fp8 vs bf16 rows) matches the oracle's
    change on the same inputs, and stays a few percent."""
    cfg16 = small("fp8w_bf16_rows", 96, 512, 8, 2, 256, w_dtype=FP8_E4M3, seed_off=63)
    cfg8 = cfg16.with_(name="fp8w_fp8_rows", fp8_dispatch=True)
    inp = make_inputs(cfg16, "cpu")
    dev = to_device(inp)
    a = gpu_layer(cfg16, dev)
    b = gpu_layer(cfg8, dev)
    gpu_delta = rel_l2(O.decode(stored(b.out), "bf16"), O.decode(stored(a.out), "bf16"))
    st = np_stored(inp)
    logits = a.logits.cpu().numpy()
    ref16 = O.layer_forward(params(cfg16), st["x"], st["w_router"], st["bias"], st["w13"],
                            st["w2"], st["w13_scale"], st["w2_scale"], logits=logits)
    ref8 = O.layer_forward(params(cfg8), st["x"], st["w_router"], st["bias"], st["w13"],
                           st["w2"], st["w13_scale"], st["w2_scale"], logits=logits)
    ora_delta = rel_l2(ref8["out"], ref16["out"])
    say(f"  fp8 vs bf16 transport: out rel-L2 GPU {gpu_delta:.4f}, oracle {ora_delta:.4f}")
    assert 0.005 < ora_delta < 0.08
    assert abs(gpu_delta - ora_delta) <= 0.2 * ora_delta


# (T, E, k): one tile; few experts in one launch; histogram + slots from the
# tile-count table (up to 256 tiles, including 1024 experts at k = 32 and few
# experts past the one-launch limit); histogram, scan and slots past 256 tiles
LAYOUT_CASES = [(200, 256, 8), (3000, 16, 4), (5000, 64, 8), (1100, 1024, 32),
                (20000, 8, 2), (33000, 256, 8), (65536, 64, 2), (70000, 64, 2)]


@pytest.mark.parametrize("T,E,k", LAYOUT_CASES, ids=[f"T{t}_E{e}_k{k}" for t, e, k in LAYOUT_CASES])
def test_dispatch_layout_paths(T, E, k):
    """Counts, offsets, the layout map and x_perm, bit for bit against the
    oracle, on every layout kernel, with a skewed expert load (a few hot
    experts) and a local range in the middle of the experts."""
    from combine_moe_route_02_amd import MoELayer
    e0, e1 = E // 4, E // 4 + max(1, E // 2)
    cfg = small(f"layout_{T}_{E}_{k}", T, 64, E, k, 128, e_begin=e0, e_end=e1,
                seed_off=70 + E % 97)
    g = torch.Generator().manual_seed(T + E + k)
    s = torch.randn((T, E), generator=g)
    bias = torch.zeros(E)
    bias[torch.randperm(E, generator=g)[:3]] = 2.0     # three hot experts
    x = torch.randn((T, 64), generator=g).to(torch.bfloat16)
    say(f"[gpu] dispatch layout T={T} E={E} k={k} local=[{e0},{e1})")
    lay = MoELayer(spec(cfg), "cuda")
    lay.logits.copy_(s.cuda())
    lay.route_from_logits(bias.cuda())
    lay.dispatch(x.cuda())
    torch.cuda.synchronize()
    st = {"x": stored(x), "bias": bias.numpy()}
    r = check_routing(cfg, lay, st)
    assert int(r["offsets"][-1]) == T * k


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_combine_rounds_like_torch(dt):
    """The float32 -> 16-bit rounding of the library's stores (here through
    combine with k = 1: out = w * y, rounded once to float32, then to the row
    type) against torch's own conversion of the same float32 product, bit for
    bit.  Inputs cover normal and subnormal 16-bit values and values near the
    format's maximum; weights give exact ties (1 + 2^-8 for bf16, 1 + 2^-11
    for f16), underflow into subnormal results and overflow to infinity.
    Only the sign of a zero result may differ (the kernel accumulates onto
    +0)."""
    from combine_moe_route_02_amd import _lib as L
    T, H = 2048, 256
    g = np.random.default_rng(BASE_SEED + 71)
    bits = g.integers(0, 1 << 16, size=(T, H), dtype=np.uint32)
    emax = 0x7F80 if dt == torch.bfloat16 else 0x7C00   # exponent all ones: inf/NaN
    sign = bits & 0x8000
    mag = bits & 0x7FFF
    mag = np.where(mag >= emax, mag - emax, mag)            # no inf or NaN inputs
    # a quarter of the rows subnormal (exponent field 0), a few near the maximum
    sub_mask = 0x007F if dt == torch.bfloat16 else 0x03FF
    rows = np.arange(T)[:, None]
    mag = np.where(rows % 4 == 1, mag & sub_mask, mag)
    mag = np.where(rows % 16 == 2, emax - 1 - (mag & 0xFF), mag)
    y16 = torch.from_numpy((sign | mag).astype(np.int32)).to(torch.int16).view(dt)
    tie = 1.0 + (2.0 ** -8 if dt == torch.bfloat16 else 2.0 ** -11)
    choices = np.array([1.0, tie, 1.0 - 2.0 ** -9, 3.0, 2.0 ** -20, 0.7], dtype=np.float32)
    w = choices[np.arange(T) % len(choices)]
    w = np.where(np.arange(T) % 7 == 6, g.uniform(-4, 4, size=T).astype(np.float32), w)
    y = y16.cuda()
    wt = torch.from_numpy(w.astype(np.float32)).cuda()
    slot = torch.arange(T, dtype=torch.int32, device="cuda").view(T, 1)
    out = torch.empty((T, H), dtype=dt, device="cuda")
    L.moe_combine(y, slot, wt.view(T, 1), out)
    torch.cuda.synchronize()
    ref = (y.float() * wt[:, None]).to(dt)
    a = out.view(torch.int16).int() & 0xFFFF
    b = ref.view(torch.int16).int() & 0xFFFF
    zero = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
    bad = (a != b) & ~zero
    say(f"  {dt}: {int(bad.sum())} of {T * H} outputs differ; "
        f"{int(torch.isinf(ref.float()).sum())} infinities, "
        f"{int(((b & emax) == 0).sum())} subnormal or zero results")
    assert int(bad.sum()) == 0
