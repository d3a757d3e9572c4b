"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: format
definitions via independent library conversions, closed forms, brute force
on tiny inputs, textbook special cases and the byte arithmetic the pages
print.  None of these tests needs a GPU.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# Codecs
# ---------------------------------------------------------------------------


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_f16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    assert _same(O.f16_decode(codes), ref)


def test_bf16_decode_exhaustive():
    codes = np.arange(65536, dtype=np.int64)
    t = torch.tensor(codes.astype(np.int16).view(np.int16)).view(torch.bfloat16)
    ref = t.to(torch.float32).numpy().astype(np.float64)
    assert _same(O.bf16_decode(codes.astype(np.uint16)), ref)


def test_e4m3_decode_exhaustive_and_named_values():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert _same(O.e4m3_decode(codes), ref)
    d = O.e4m3_decode(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x80, 0xFE],
                               dtype=np.uint8))
    assert list(d[:5]) == [448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0]
    assert d[5] == 0 and np.signbit(d[5]) and d[6] == -448.0
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def _random_f64(n):
    mant = rng.uniform(1.0, 2.0, n)
    exps = rng.integers(-150, 130, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, exps)


def test_round_f32_matches_hardware_conversion():
    x = _random_f64(200000)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    assert _same(O.round_rne(x, O.F32), ref)


def test_round_f16_matches_numpy_double_to_half():
    x = np.concatenate([_random_f64(100000) * 2.0 ** -100,   # mostly tiny/zero
                        rng.normal(0, 1000, 100000),
                        rng.normal(0, 1e-5, 100000)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert _same(O.round_rne(x, O.F16), ref)


def test_round_bf16_matches_torch_on_float32_inputs():
    x = rng.normal(0, 3, 200000).astype(np.float32)
    x[:1000] = np.ldexp(rng.uniform(1, 2, 1000), rng.integers(-140, -120, 1000))
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert _same(O.round_rne(x.astype(np.float64), O.BF16), ref)


def test_round_bf16_edge_cases_from_the_definition():
    u = 2.0 ** -7                              # bf16 spacing at 1.0
    cases = {
        1 + u / 2: 1.0,                        # tie -> even (1.0)
        1 + 3 * u / 2: 1 + 2 * u,              # tie -> even mantissa
        1 + u / 2 + 2.0 ** -40: 1 + u,         # just above the tie: up
        1 + u / 2 - 2.0 ** -40: 1.0,           # just below the tie: down
        2.0 ** -133: 2.0 ** -133,              # smallest subnormal
        2.0 ** -134: 0.0,                      # half of it: tie -> 0 (even)
        1.5 * 2.0 ** -134: 2.0 ** -133,
        (2 - u) * 2.0 ** 127: (2 - u) * 2.0 ** 127,   # largest finite
        (2 - u / 2) * 2.0 ** 127: math.inf,           # its tie with 2**128
        -0.0: -0.0,
    }
    for x, want in cases.items():
        got = float(O.round_rne(np.float64(x), O.BF16))
        assert got == want and math.copysign(1, got) == math.copysign(1, want), x
    # encode/decode round trip of every finite bf16 value
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_decode(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(O.bf16_encode(vals[fin]), codes[fin])


def test_f16_encode_round_trip_all_finite_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.f16_decode(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(O.f16_encode(vals[fin]), codes[fin])


# ---------------------------------------------------------------------------
# Router logits
# ---------------------------------------------------------------------------


def test_router_logits_brute_force():
    T, H, E = 5, 7, 3
    x = rng.normal(size=(T, H)).astype(np.float32).astype(np.float64)
    w = rng.normal(size=(E, H)).astype(np.float32).astype(np.float64)
    got = O.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            exact = math.fsum(x[t, h] * w[e, h] for h in range(H))
            assert got[t, e] == np.float32(exact)
    assert got.dtype == np.float32


def test_router_logits_identity_router_returns_inputs():
    x = rng.normal(size=(6, 8)).astype(np.float32).astype(np.float64)
    w = np.eye(8)[:5]
    assert np.array_equal(O.router_logits(x, w), x[:, :5].astype(np.float32))


# ---------------------------------------------------------------------------
# Top-k selection and gate weights
# ---------------------------------------------------------------------------


def _brute_topk(s_row, k):
    """Repeatedly take the largest remaining score, lowest index on ties."""
    left = list(range(len(s_row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if s_row[e] > s_row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8, 16])
def test_topk_brute_force_with_mass_ties(E):
    T = 150
    s = rng.integers(-1, 2, size=(T, E)).astype(np.float32)
    s[rng.random((T, E)) < 0.2] = -0.0        # signed zeros tie with +0.0
    for k in range(1, E + 1):
        idx = O.topk_select(s, k)
        for t in range(T):
            assert list(idx[t]) == _brute_topk(list(s[t]), k)


def test_topk_k1_is_first_argmax_and_kE_is_stable_descending_sort():
    s = rng.integers(-3, 4, size=(300, 12)).astype(np.float32)
    assert np.array_equal(O.topk_select(s, 1)[:, 0], np.argmax(s, axis=1))
    full = O.topk_select(s, 12)
    for t in range(300):
        assert list(full[t]) == sorted(range(12), key=lambda e: (-s[t, e], e))


def test_signed_zero_is_a_tie():
    s = np.array([[-0.0, 0.0], [0.0, -0.0]], dtype=np.float32)
    assert O.topk_select(s, 2).tolist() == [[0, 1], [0, 1]]


def test_selection_adds_bias_in_float32():
    logits = np.array([[1.0, 2.0, 3.0]], np.float32)
    bias = np.array([5.0, 0.0, 0.0], np.float32)
    s = O.selection_scores(logits, bias)
    assert s.dtype == np.float32 and O.topk_select(s, 1)[0, 0] == 0
    # float32 addition, not float64: 1 + 2**-30 is 1 in float32
    s2 = O.selection_scores(np.array([[1.0]], np.float32),
                            np.array([2.0 ** -30], np.float32))
    assert s2[0, 0] == 1.0


def test_softmax_two_experts_closed_form():
    a, b = 0.7, -1.3
    s = np.array([[a, b]], np.float32)
    idx, w = O.route(s, None, 1, "softmax", False)
    assert idx[0, 0] == 0
    want = 1.0 / (1.0 + math.exp(float(np.float32(b)) - float(np.float32(a))))
    assert w[0, 0] == np.float32(want)


def test_softmax_brute_force_and_temperature():
    s = rng.normal(size=(20, 6)).astype(np.float32)
    for inv_t in (1.0, 1 / 0.3, 0.5):
        idx, w = O.route(s, None, 3, "softmax", False, inv_t)
        for t in range(20):
            z = [math.exp(inv_t * float(v)) for v in s[t]]
            tot = math.fsum(z)
            for j in range(3):
                want = z[idx[t, j]] / tot
                assert abs(w[t, j] - want) <= 2 ** -23 * want


def test_softmax_weights_sum_to_one_over_all_experts():
    s = rng.normal(size=(50, 8)).astype(np.float32)
    _, w = O.route(s, None, 8, "softmax", False)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=8 * 2 ** -24)


def test_zero_inverse_temperature_gives_uniform_weights():
    s = rng.normal(size=(10, 8)).astype(np.float32)
    _, w = O.route(s, None, 2, "softmax", False, 0.0)
    assert np.all(w == np.float32(1 / 8))


def test_sigmoid_closed_forms():
    s = np.array([[0.0, math.log(3.0), -math.log(3.0)]], np.float32)
    idx, w = O.route(s, None, 3, "sigmoid", False)
    assert idx.tolist() == [[1, 0, 2]]
    want = [1 / (1 + math.exp(-float(np.float32(math.log(3.0))))), 0.5,
            1 / (1 + math.exp(float(np.float32(math.log(3.0)))))]
    assert np.array_equal(w[0], np.array(want, np.float32))


def test_renormalised_weights():
    s = rng.normal(size=(40, 16)).astype(np.float32)
    for gate in ("softmax", "sigmoid"):
        _, w = O.route(s, None, 4, gate, True)
        assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=4 * 2 ** -24)
        _, w1 = O.route(s, None, 1, gate, True)
        assert np.all(w1 == 1.0)


# Minimum-probability threshold (GPT-4 MoE page, section 2.3 stage 2 and the
# section 4.1 sketch): a pick survives only if its probability is above it.


def _py_softmax(row, inv_t):
    m = max(float(v) for v in row)
    z = [math.exp((float(v) - m) * inv_t) for v in row]
    tot = math.fsum(z)
    return [v / tot for v in z]


@pytest.mark.parametrize("inv_t,theta,renorm", [(1 / 0.3, 0.05, False), (1.0, 0.15, True),
                                                (0.5, 0.12, False), (1 / 0.3, 0.05, True)])
def test_threshold_brute_force(inv_t, theta, renorm):
    """Plain Python per token: the k best experts by (score desc, index asc),
    kept iff their probability is above theta, renormalised over the kept."""
    r = np.random.default_rng(77)
    T, E, k = 60, 6, 3
    s = r.normal(size=(T, E)).astype(np.float32)
    idx, w = O.route(s, None, k, "softmax", renorm, inv_t, theta)
    n_drop = 0
    for t in range(T):
        p = _py_softmax(s[t], inv_t)
        order = sorted(range(E), key=lambda e: (-float(s[t, e]), e))[:k]
        assert all(abs(p[e] - theta) > 1e-9 for e in order)
        kept = [e for e in order if p[e] > theta]
        tot = math.fsum(p[e] for e in kept)
        for j in range(k):
            if j < len(kept):
                e = kept[j]
                assert idx[t, j] == e
                want = p[e] / tot if renorm else p[e]
                assert abs(float(w[t, j]) - want) <= 2 ** -23 * want
            else:
                assert idx[t, j] == -1 and w[t, j] == 0.0
        n_drop += k - len(kept)
    assert 0 < n_drop < T * k      # both outcomes occur


def test_threshold_with_k_equal_E_is_the_set_above_it():
    """k = E: the kept picks are exactly {e : softmax_e > theta} (library
    softmax), in descending score order, and every other slot is -1."""
    from scipy.special import softmax
    r = np.random.default_rng(78)
    s = r.normal(size=(50, 8)).astype(np.float32)
    theta = 0.11
    idx, _ = O.route(s, None, 8, "softmax", False, 1.0, theta)
    p = softmax(s.astype(np.float64), axis=1)
    for t in range(50):
        want = [int(e) for e in np.argsort(-s[t].astype(np.float64), kind="stable")
                if p[t, e] > theta]
        got = idx[t].tolist()
        assert got == want + [-1] * (8 - len(want))


def test_threshold_sigmoid_closed_form():
    s = np.array([[0.0, math.log(3.0), -math.log(3.0)]], np.float32)
    idx, w = O.route(s, None, 3, "sigmoid", True, 1.0, 0.4)
    assert idx.tolist() == [[1, 0, -1]]
    a = 1 / (1 + math.exp(-float(np.float32(math.log(3.0)))))   # 0.75 up to f32 input
    assert w[0, 0] == np.float32(a / (a + 0.5))
    assert w[0, 1] == np.float32(0.5 / (a + 0.5)) and w[0, 2] == 0.0


def test_threshold_zero_is_off_and_one_drops_every_softmax_pick():
    r = np.random.default_rng(79)
    s = r.normal(size=(30, 8)).astype(np.float32)
    a = O.route(s, None, 3, "softmax", True, 1.0)
    b = O.route(s, None, 3, "softmax", True, 1.0, 0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    idx, w = O.route(s, None, 3, "softmax", True, 1.0, 1.0)
    assert np.all(idx == -1) and np.all(w == 0.0)
    counts = O.expert_counts(idx, 8)
    off = O.expert_offsets(counts)
    assert np.all(counts == 0) and np.all(off == 0)
    slot_of, row_token = O.layout_map(idx, off)
    assert np.all(slot_of == -1) and np.all(row_token == -1)
    out = O.combine(np.ones((90, 4)), slot_of, w, O.F32)
    assert np.all(out == 0.0)


def test_dispatch_and_combine_with_dropped_picks():
    """Counts = bincount of the kept picks; the layout is the stable argsort of
    the kept (expert, token) pairs; combine adds only kept picks."""
    r = np.random.default_rng(80)
    T, E, k, H = 200, 8, 4, 6
    s = r.normal(size=(T, E)).astype(np.float32)
    idx, w = O.route(s, None, k, "softmax", False, 1 / 0.3, 0.05)
    keep = idx >= 0
    assert 0 < keep.sum() < T * k
    assert np.all(np.diff(keep.astype(np.int8), axis=1) <= 0)    # dropped = a suffix
    counts = O.expert_counts(idx, E)
    assert np.array_equal(counts, np.bincount(idx[keep], minlength=E))
    off = O.expert_offsets(counts)
    assert off[E] == keep.sum()
    slot_of, row_token = O.layout_map(idx, off)
    tt, jj = np.nonzero(keep)
    order = np.argsort(idx[tt, jj].astype(np.int64) * T + tt, kind="stable")
    n = int(keep.sum())
    assert np.array_equal(row_token[:n], tt[order]) and np.all(row_token[n:] == -1)
    inv = np.empty(n, np.int64)
    inv[order] = np.arange(n)
    assert np.array_equal(slot_of[tt, jj], inv) and np.all(slot_of[~keep] == -1)
    y = r.normal(size=(T * k, H))
    out = O.combine(y, slot_of, w, O.F32)
    for t in range(0, T, 7):
        for c in range(H):
            acc = 0.0
            for j in range(k):
                if idx[t, j] >= 0:
                    acc += float(w[t, j]) * y[slot_of[t, j], c]
            assert out[t, c] == np.float32(acc)


# fp8 transport of the dispatched rows (ThunderEP page, section 3.3)


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    fin = codes[~np.isnan(O.e4m3_decode(codes))]
    assert len(fin) == 254
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(fin)), fin)


def test_e4m3_encode_ties_to_even_and_matches_torch():
    """Every midpoint between adjacent finite magnitudes goes to the code with
    an even mantissa; random values agree with torch's float8_e4m3fn cast."""
    pos = np.arange(0, 0x7F, dtype=np.uint8)          # 0 .. 448 ascending
    v = O.e4m3_decode(pos)
    mid = (v[:-1] + v[1:]) / 2
    got = O.e4m3_encode(mid)
    want = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, want)
    assert np.array_equal(O.e4m3_encode(-mid), want | 0x80)
    x = np.concatenate([mid, rng.uniform(-448, 448, 20000), rng.normal(size=20000) * 1e-2])
    t = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), t)


def test_e4m3_encode_saturates_and_keeps_sign():
    got = O.e4m3_encode([464.0, 470.0, 1e9, -1e9, 0.0, -0.0, -1e-9, 2.0 ** -10,
                         3 * 2.0 ** -10, float("nan")])
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80, 0x00, 0x02, 0x7F]


def test_row_exponent_closed_form():
    amax = [448.0, np.nextafter(448.0, 1e9), 224.0, np.nextafter(224.0, 1e9), 1.0,
            0.0, 2.0 ** -133, 3.0e38]
    got = O.e4m3_row_exponent(amax).tolist()
    assert got == [0, 1, -1, 0, -8, 0, -141, 120]
    for a, e in zip(amax[:5] + amax[6:], got[:5] + got[6:]):
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)


def test_row_quantisation_scales_and_codes():
    """Per-row power-of-two scales put each row's amax in (224, 448]; the codes
    are the library's float8_e4m3fn cast of the exactly scaled row."""
    r = np.random.default_rng(81)
    mags = 10.0 ** r.uniform(-30, 30, size=64)
    x = O.bf16_decode(O.bf16_encode(r.normal(size=(64, 96)) * mags[:, None]))
    x[5] = 0.0
    codes, sc = O.quantize_rows_e4m3(x)
    e = np.log2(sc.astype(np.float64))
    assert np.all(e == np.round(e))                       # powers of two
    amax = np.abs(x).max(axis=1)
    ratio = amax[amax > 0] / sc[amax > 0]
    assert np.all((ratio > 224) & (ratio <= 448))
    assert sc[5] == 1.0 and np.all(codes[5] == 0)
    t = torch.tensor(np.ldexp(x, -e.astype(np.int64)[:, None])).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, t.view(torch.uint8).numpy())
    deq = O.e4m3_decode(codes) * sc.astype(np.float64)[:, None]
    # half a step of 3 mantissa bits, or half the subnormal quantum 2^-9 * scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sc.astype(np.float64)[:, None])
    assert np.all(np.abs(deq - x) <= bound)


# ---------------------------------------------------------------------------
# Dispatch
# ---------------------------------------------------------------------------


def _random_routing(T, E, k, seed=0):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 2), (255, 16, 4),
                                   (256, 8, 8), (1000, 64, 6)])
def test_dispatch_against_bincount_cumsum_and_stable_argsort(T, E, k):
    idx = _random_routing(T, E, k, seed=T + E + k)
    counts = O.expert_counts(idx, E)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    off = O.expert_offsets(counts)
    assert off[0] == 0 and off[E] == T * k
    assert np.array_equal(off[1:], np.cumsum(counts))
    slot_of, row_token = O.layout_map(idx, off)
    # textbook: stable sort of the pairs by key e*T + t
    t_of = np.repeat(np.arange(T), k)
    order = np.argsort(idx.ravel().astype(np.int64) * T + t_of, kind="stable")
    assert np.array_equal(row_token, t_of[order])
    inv = np.empty(T * k, np.int64)
    inv[order] = np.arange(T * k)
    assert np.array_equal(slot_of.ravel(), inv)


def test_layout_invariants_with_skew():
    T, E, k = 500, 8, 2
    idx = _random_routing(T, E, k, 3)
    idx[: T // 2, 0] = 5                       # hot expert
    idx[: T // 2, 1] = np.where(idx[: T // 2, 1] == 5, 6, idx[: T // 2, 1])
    counts = O.expert_counts(idx, E)
    off = O.expert_offsets(counts)
    slot_of, row_token = O.layout_map(idx, off)
    assert sorted(slot_of.ravel().tolist()) == list(range(T * k))   # bijection
    for t in range(T):
        for j in range(k):
            r = slot_of[t, j]
            assert row_token[r] == t and off[idx[t, j]] <= r < off[idx[t, j] + 1]
    for e in range(E):
        seg = row_token[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)        # ascending token order
    assert np.array_equal(np.bincount(row_token, minlength=T), np.full(T, k))


def test_gather_is_a_bit_copy():
    x = rng.integers(0, 65536, size=(10, 16)).astype(np.uint16)
    idx = _random_routing(10, 4, 2, 9)
    off = O.expert_offsets(O.expert_counts(idx, 4))
    slot_of, row_token = O.layout_map(idx, off)
    xp = O.gather_rows(x, row_token, 0, 20)
    for t in range(10):
        for j in range(2):
            assert np.array_equal(xp[slot_of[t, j]], x[t])


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------


def test_activation_known_values():
    # Phi(1) and Phi(-1) of the standard normal (textbook table values)
    assert abs(O.gelu_erf(np.array(1.0)) - 0.8413447460685429) < 1e-15
    assert abs(O.gelu_erf(np.array(-1.0)) + 0.15865525393145707) < 1e-15
    assert O.gelu_erf(np.array(0.0)) == 0.0
    assert abs(O.silu(np.array(1.0)) - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(O.silu(np.array(-2.0)) + 2 / (1 + math.exp(2))) < 1e-16


def test_swiglu_expert_brute_force():
    H, I, R = 5, 3, 4
    X = rng.normal(size=(R, H))
    w13 = rng.normal(size=(2 * I, H))
    w2 = rng.normal(size=(H, I))
    y = O.expert_ffn(X, w13, w2, "swiglu", O.F32)
    for r in range(R):
        h = []
        for i in range(I):
            g = math.fsum(X[r, c] * w13[i, c] for c in range(H))
            u = math.fsum(X[r, c] * w13[I + i, c] for c in range(H))
            h.append(float(np.float32(g / (1 + math.exp(-g)) * u)))
        for o in range(H):
            want = np.float32(math.fsum(h[i] * w2[o, i] for i in range(I)))
            assert abs(y[r, o] - want) <= 2 ** -22 * max(abs(want), 1e-30)


def test_gelu_expert_brute_force():
    H, I, R = 4, 6, 3
    X = rng.normal(size=(R, H))
    w1 = rng.normal(size=(I, H))
    w2 = rng.normal(size=(H, I))
    y = O.expert_ffn(X, w1, w2, "gelu", O.F32)
    for r in range(R):
        h = []
        for i in range(I):
            a = math.fsum(X[r, c] * w1[i, c] for c in range(H))
            h.append(float(np.float32(0.5 * a * (1 + math.erf(a / math.sqrt(2))))))
        for o in range(H):
            want = np.float32(math.fsum(h[i] * w2[o, i] for i in range(I)))
            assert abs(y[r, o] - want) <= 2 ** -22 * max(abs(want), 1e-30)


def test_fp8_block_dequant_uses_row_block_then_column_block():
    codes = np.full((256, 384), 0x38, np.uint8)            # every code = 1.0
    scales = np.array([[2.0 ** (i + 3 * j) for j in range(3)] for i in range(2)])
    w = O.dequant_e4m3_blocks(codes, scales)
    for n in (0, 127, 128, 255):
        for c in (0, 127, 128, 300):
            assert w[n, c] == 2.0 ** (n // 128 + 3 * (c // 128))
    codes[5, 7] = 0x7E                                    # 448
    assert O.dequant_e4m3_blocks(codes, scales)[5, 7] == 448.0


# ---------------------------------------------------------------------------
# Placement of replicated experts and load statistics (TensorRT-LLM
# large-EP page, high-level design)
# ---------------------------------------------------------------------------


def test_identity_placement_is_the_identity():
    idx = _random_routing(50, 8, 3, 4)
    idx[::7, 2] = -1
    out = O.place_experts(idx, np.arange(9), np.arange(8))
    assert np.array_equal(out, idx)


def test_placement_spreads_an_expert_over_its_copies_in_token_order():
    """Every token picks expert 0, which has n copies: copy r serves tokens
    r, r + n, ... (ceil((T - r) / n) of them); other experts keep one copy."""
    T, n = 103, 4
    idx = np.zeros((T, 1), np.int32)
    rep_off = np.array([0, n, n + 1])
    rep_phys = np.array([5, 0, 2, 7, 1])
    out = O.place_experts(idx, rep_off, rep_phys)
    for r, p in enumerate(rep_phys[:n]):
        assert np.array_equal(np.nonzero(out[:, 0] == p)[0], np.arange(r, T, n))
        assert (out == p).sum() == -(-(T - r) // n)


def test_placement_conserves_every_logical_load():
    r = np.random.default_rng(82)
    T, E, k = 400, 16, 4
    idx = _random_routing(T, E, k, 11)
    idx[r.random((T, k)) < 0.1] = -1
    ncopy = r.integers(1, 4, size=E)
    rep_off = np.concatenate([[0], np.cumsum(ncopy)])
    rep_phys = r.permutation(int(ncopy.sum())).astype(np.int32)
    phys = O.place_experts(idx, rep_off, rep_phys)
    assert np.array_equal(phys < 0, idx < 0)
    pload = O.expert_counts(phys, int(ncopy.sum()))
    lload = O.expert_load(idx, E)
    assert np.array_equal(lload, np.bincount(idx[idx >= 0], minlength=E).astype(np.uint64))
    for e in range(E):
        assert pload[rep_phys[rep_off[e]:rep_off[e + 1]]].sum() == lload[e]
    for t in range(0, T, 13):                  # brute force, one pick at a time
        for j in range(k):
            e = idx[t, j]
            if e >= 0:
                assert phys[t, j] == rep_phys[rep_off[e] + t % ncopy[e]]


def test_replicated_layer_equals_the_unreplicated_layer():
    """Copies hold their expert's weights, so routing picks to copies changes
    no output (the float64 sums are the same numbers in the same order)."""
    r = np.random.default_rng(83)
    p = O.LayerParams(T=40, H=16, E=4, k=2, I=8, act_dtype=O.F32, w_dtype=O.F32,
                      gate="softmax", renorm=False, act="swiglu", e_begin=0, e_end=4)
    x = r.normal(size=(40, 16)).astype(np.float32)
    wr = (r.normal(size=(4, 16)) / 4).astype(np.float32)
    w13 = (r.normal(size=(4, 16, 16)) / 4).astype(np.float32)
    w2 = (r.normal(size=(4, 16, 8)) / 3).astype(np.float32)
    base = O.layer_forward(p, x, wr, None, w13, w2)
    ncopy = np.array([1, 3, 1, 2])
    rep_off = np.concatenate([[0], np.cumsum(ncopy)])
    rep_phys = np.array([0, 1, 4, 5, 2, 3, 6], np.int32)
    owner = np.empty(7, np.int64)
    for e in range(4):
        owner[rep_phys[rep_off[e]:rep_off[e + 1]]] = e
    pp = O.LayerParams(**{**p.__dict__, "e_end": 7})
    rep = O.layer_forward(pp, x, wr, None, w13[owner], w2[owner],
                          placement=(rep_off, rep_phys, 7))
    assert np.array_equal(rep["out"], base["out"])
    assert np.array_equal(rep["topk_idx"], base["topk_idx"])
    assert sorted(np.unique(rep["topk_phys"]).tolist()) == list(range(7))


# ---------------------------------------------------------------------------
# Combine and the whole layer
# ---------------------------------------------------------------------------


def test_combine_brute_force():
    T, k, H, N = 6, 3, 5, 18
    y = rng.normal(size=(N, H))
    slot_of = rng.permutation(N)[: T * k].reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    out = O.combine(y, slot_of, w, O.F32)
    for t in range(T):
        for c in range(H):
            acc = 0.0
            for j in range(k):
                acc += float(w[t, j]) * y[slot_of[t, j], c]
            assert out[t, c] == np.float32(acc)


def test_combine_top1_renormalised_is_the_inverse_permutation():
    T, E = 64, 8
    s = rng.normal(size=(T, E)).astype(np.float32)
    idx, w = O.route(s, None, 1, "softmax", True)
    off = O.expert_offsets(O.expert_counts(idx, E))
    slot_of, _ = O.layout_map(idx, off)
    y = O.bf16_decode(rng.integers(0, 0x7F00, size=(T, 32)).astype(np.uint16))
    out = O.combine(y, slot_of, w, O.BF16)
    assert np.array_equal(out, y[slot_of[:, 0]])


def test_dispatch_combine_round_trip_returns_tokens():
    """Dispatch then combine with y := x_perm and weights summing to one."""
    T, E, k, H = 128, 16, 4, 64
    s = rng.normal(size=(T, E)).astype(np.float32)
    idx, w = O.route(s, None, k, "softmax", True)
    off = O.expert_offsets(O.expert_counts(idx, E))
    slot_of, row_token = O.layout_map(idx, off)
    x_bits = O.bf16_encode(rng.normal(size=(T, H)))
    xp = O.gather_rows(x_bits, row_token, 0, T * k)
    out = O.combine(O.bf16_decode(xp), slot_of, w, O.BF16)
    x = O.bf16_decode(x_bits)
    assert np.all(np.abs(out - x) <= np.abs(x) * 2.0 ** -8 + 1e-30)


def test_single_expert_layer_is_a_dense_ffn():
    """E = 1, k = 1, renormalised: the layer reduces to y = FFN(x)."""
    T, H, I = 32, 16, 24
    p = O.LayerParams(T=T, H=H, E=1, k=1, I=I, act_dtype=O.BF16, w_dtype=O.BF16,
                      gate="softmax", renorm=True, act="swiglu", e_begin=0, e_end=1)
    xb = O.bf16_encode(rng.normal(size=(T, H)))
    wr = O.bf16_encode(rng.normal(size=(1, H)))
    w13 = O.bf16_encode(rng.normal(size=(1, 2 * I, H)) / 4)
    w2 = O.bf16_encode(rng.normal(size=(1, H, I)) / 5)
    res = O.layer_forward(p, xb, wr, None, w13, w2)
    # independent dense evaluation with torch float64
    X = torch.tensor(O.bf16_decode(xb))
    W13 = torch.tensor(O.bf16_decode(w13[0]))
    W2 = torch.tensor(O.bf16_decode(w2[0]))
    g, u = X @ W13[:I].T, X @ W13[I:].T
    h = torch.tensor(O.bf16_decode(O.bf16_encode((torch.nn.functional.silu(g) * u).numpy())))
    y = O.bf16_decode(O.bf16_encode((h @ W2.T).numpy()))
    assert res["topk_w"].tolist() == [[1.0]] * T
    assert np.array_equal(res["out"], y)


def test_layer_uses_remote_rows_for_non_local_experts():
    T, H, E, k, I = 16, 8, 4, 2, 8
    p = O.LayerParams(T=T, H=H, E=E, k=k, I=I, act_dtype=O.BF16, w_dtype=O.BF16,
                      gate="sigmoid", renorm=False, act="swiglu", e_begin=0, e_end=2)
    xb = O.bf16_encode(rng.normal(size=(T, H)))
    wr = O.bf16_encode(rng.normal(size=(E, H)))
    w13 = O.bf16_encode(rng.normal(size=(2, 2 * I, H)))
    w2 = O.bf16_encode(rng.normal(size=(2, H, I)))
    yr = O.bf16_encode(rng.normal(size=(T * k, H)))
    res = O.layer_forward(p, xb, wr, None, w13, w2, y_remote_stored=yr)
    r1 = res["offsets"][2]
    assert np.array_equal(res["y_perm"][r1:], O.bf16_decode(yr)[r1:])
    assert res["x_perm"].shape == (r1, H)


# ---------------------------------------------------------------------------
# The pages' byte arithmetic
# ---------------------------------------------------------------------------


def test_thunderep_layer_bytes():
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["thunderep_bytes"]
    B, E = g["B"], g["experts"]
    idx = (np.arange(B) % E).astype(np.int32)[:, None]   # top-1, half remote
    counts = O.expert_counts(idx, E)
    per_dir = O.a2a_bytes_per_direction(counts, g["remote_experts"], g["H"],
                                        g["elem_bytes"])
    assert per_dir == B // 2 * g["H"] * g["elem_bytes"] == 16 * 2 ** 20
    layer = 4 * per_dir                       # 2 phases x 2 directions
    assert layer == g["layer_MB_approx"] * 2 ** 20
    forward = layer * g["layers"]
    assert forward == g["forward_GB_approx"] * 2 ** 30
    ms = forward / (2 * g["pcie_GBps_per_direction"] * 1e9) * 1e3
    assert abs(ms - g["ideal_ms_approx"]) / g["ideal_ms_approx"] < 0.1


def test_trtllm_fp4_expert_bytes():
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["trtllm_fp4_expert"]
    # 4-bit values with one 1-byte scale per 16 values, DeepSeek-R1 expert dims
    b = O.expert_weight_bytes(7168, 2048, 4, block_elems=16, scale_bytes=1)
    assert round(b / 2 ** 20) == g["expert_MiB"]
    assert (g["expert_MiB"] * 2 ** 20 * g["experts_per_layer"] * g["moe_layers"]
            == g["total_GiB"] * 2 ** 30)
    # the fp8 block-scaled experts of the decode layer: e4m3 + f32 per 128x128
    assert O.expert_weight_bytes(7168, 2048, 8, 128 * 128, 4) == 44_050_944
