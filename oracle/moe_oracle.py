"""Plain CPU oracle for the MoE-layer forward (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never calls it.  It shares no code with
the HIP library: it has its own codecs (IEEE binary16, bfloat16, OCP E4M3FN),
accumulates in float64 and stores each result in the precision the layer
fixes.

What it computes, step by step, with the passage each step follows:

1. Router logits, one score per expert for each token
   (ThunderEP page, section 1.1: a router scores each token and picks the
   top-1 or top-2 experts; GPT-4 MoE page, section 2.3 stage 1: a small
   router network emits one logit per expert).
2. Top-k selection by score, ties broken towards the lower expert index,
   then the gate weights: softmax over all experts (optionally divided by a
   temperature) evaluated at the picks, or a sigmoid of the picked scores,
   optionally renormalised to sum 1 (GPT-4 MoE page, section 4.1 step 2
   sketch: softmax over all experts, then top-k, weights = the selected
   probabilities; section 2.3 and the xDeepServe diary section 5.3 for the
   temperature, default 1.0).  With a minimum-probability threshold (GPT-4
   MoE page, section 2.3 stage 2, and the same sketch's mask) a pick whose
   gate value is not above it is dropped: index -1, weight 0, no layout row,
   nothing to combine.
3. Dispatch: per-expert counts, their exclusive prefix sum, and a dense
   expert-contiguous layout in which each token is written once per chosen
   expert (DySHARP page, section 1: dispatch sends one token to its k
   experts; section 3.1 item 3: the algebraic-to-layout index table with
   incremental dense allocation, reused in reverse by combine; ThunderEP
   page, sections 3.4 and 5.2: tokens for one expert gathered into one
   contiguous buffer).
4. Expert FFN on each local expert's rows (GPT-4 MoE page, section 3.1
   table: Linear -> GELU -> Linear; the gated SwiGLU form of the larger
   layer shapes).
5. Combine: the gate-weighted sum of a token's k expert outputs, back in
   token order (DySHARP page, section 1: k results reduced into one;
   ThunderEP page, section 2.1: the weighted sum at combine).

Where the pages leave a step open, the reading taken is the plainest one the
rest supports: selection uses the bias-added float32 scores (softmax and
sigmoid are monotone, so this equals selecting by probability without ties
created by rounding); the k outputs are ordered by descending score then
ascending index; rows inside an expert's segment are in ascending token
order; h and y are rounded once to the activation dtype; combine sums in
pick order and rounds once.

Every function here is pinned by the CPU tests against closed forms, brute
force on tiny inputs, library routines for the special cases that reduce to
them, and the byte arithmetic printed on the pages.
"""

from __future__ import annotations

import math
import time
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

try:  # exact erf, vectorised
    from scipy.special import erf as _erf
except Exception:  # pragma: no cover - scipy is present in this image
    _erf = np.vectorize(math.erf)

F32, F16, BF16, FP8_E4M3 = "f32", "f16", "bf16", "e4m3"

# ---------------------------------------------------------------------------
# Codecs, written from the format definitions
# ---------------------------------------------------------------------------

# (significand bits including the implicit one, minimum normal exponent,
#  maximum exponent) of the IEEE-style binary formats used by the layer.
_FORMATS = {
    F32: (24, -126, 127),
    F16: (11, -14, 15),
    BF16: (8, -126, 127),
}


def round_rne(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    Subnormals are kept (the quantum stops shrinking below the minimum
    normal exponent); magnitudes whose rounded value exceeds the largest
    finite number become infinities, as IEEE 754 round-to-nearest requires.
    Returns float64 values that are exactly representable in ``fmt``.
    """
    p, emin, emax = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)                 # ax = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)         # unbiased exponent, clamped at emin
    q = np.ldexp(1.0, e - (p - 1))       # spacing of fmt numbers near ax
    r = np.round(ax / q) * q             # np.round: halves go to even
    max_finite = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    r = np.where(r > max_finite, np.inf, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bfloat16 is the top half of binary32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (RNE)."""
    r = round_rne(x, BF16).astype(np.float32)   # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f16_decode(bits: np.ndarray) -> np.ndarray:
    """IEEE 754 binary16 bit patterns -> float64."""
    b = np.asarray(bits).astype(np.int64)
    s = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m, -24), np.ldexp(1024.0 + m, e - 25))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return s * val


def f16_encode(x) -> np.ndarray:
    """float64 -> binary16 bit patterns (RNE)."""
    r = round_rne(x, F16)
    return r.astype(np.float16).view(np.uint16)  # exact: r is a binary16 value


def e4m3_decode(bits: np.ndarray) -> np.ndarray:
    """OCP 8-bit E4M3 ("E4M3FN": bias 7, no infinities) codes -> float64.

    exponent field 0 -> subnormal m * 2**-9; S.1111.111 -> NaN; otherwise
    (1 + m/8) * 2**(e-7).
    """
    b = np.asarray(bits).astype(np.int64)
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m, -9), np.ldexp(8.0 + m, e - 10))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """float64 -> OCP E4M3FN codes, round to nearest even, saturating to +-448.

    Written from the format: 4 significant bits, smallest normal exponent -6
    (subnormals are multiples of 2**-9), largest finite 1.75 * 2**8 = 448
    (the pattern S.1111.111 is NaN).  The sign bit follows the input's sign,
    so -0.0 and negative values that round to zero give 0x80.  NaN -> 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # exponent, clamped at the subnormal range
    q = np.ldexp(1.0, e - 3)                  # spacing of E4M3 values near a
    r = np.minimum(np.round(a / q) * q, E4M3_MAX)   # np.round: halves to even
    sub = r < 2.0 ** -6
    _, er = np.frexp(np.where(sub, 1.0, r))
    E = er - 1                                # exponent of a normal result
    mant = np.where(sub, 0, np.round(np.ldexp(r, -E) * 8.0) - 8.0)
    code = np.where(sub, np.round(np.ldexp(r, 9)), ((E + 7) << 3) + mant)
    code = code.astype(np.int64) | (np.signbit(x).astype(np.int64) << 7)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def e4m3_row_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2**e (0 where amax == 0).

    448 = 0.875 * 2**9 and amax = m * 2**ex with m in [0.5, 1), so
    e = ex - 9, plus one when m > 0.875; exact, no logarithms.
    """
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)
    e = ex - 9 + (m > 0.875)
    return np.where(amax > 0, e, 0).astype(np.int64)


def quantize_rows_e4m3(x: np.ndarray):
    """fp8 transport of activation rows (ThunderEP page, section 3.3: send the
    dispatched activations as 8-bit floats with a dynamic scale).  Each row
    gets the power-of-two scale 2**e of e4m3_row_exponent(max |x|), so that
    x * 2**-e is exact and within +-448; codes are e4m3_encode of it.

    Returns (codes uint8 [R, H], scales float32 [R] = 2**e).
    """
    x = np.asarray(x, dtype=np.float64)
    e = e4m3_row_exponent(np.abs(x).max(axis=1) if x.shape[1] else np.zeros(len(x)))
    codes = e4m3_encode(np.ldexp(x, -e[:, None]))
    return codes, np.ldexp(1.0, e).astype(np.float32)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bits for 16/8-bit formats, float32 values) -> float64."""
    if dtype == F32:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_decode(arr)
    if dtype == F16:
        return f16_decode(arr)
    if dtype == FP8_E4M3:
        return e4m3_decode(arr)
    raise ValueError(dtype)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> stored form of ``dtype`` (float32 values or bit patterns)."""
    if dtype == F32:
        return round_rne(x, F32).astype(np.float32)
    if dtype == BF16:
        return bf16_encode(x)
    if dtype == F16:
        return f16_encode(x)
    raise ValueError(dtype)


def round_act(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the activation dtype, keeping float64 storage."""
    return round_rne(x, dtype)


# ---------------------------------------------------------------------------
# 1. Router logits
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h], summed in float64, stored f32.

    ``x`` [T, H] and ``w_router`` [E, H] are float64 values of the stored
    activations and router weights.
    """
    return round_rne(x @ w_router.T, F32).astype(np.float32)


# ---------------------------------------------------------------------------
# 2. Top-k gating
# ---------------------------------------------------------------------------


def selection_scores(logits: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """s = logits + bias, one float32 addition (IEEE RNE), as float32."""
    s = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        s = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return s


def topk_select(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per token, descending; ties -> lower index.

    A stable sort of -s keeps equal scores in ascending index order, and
    -0.0 and +0.0 compare equal, so they tie as IEEE equality says.
    """
    order = np.argsort(-s.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def raw_gate(s: np.ndarray, idx: np.ndarray, gate: str,
             inv_temperature: float = 1.0) -> np.ndarray:
    """Gate value of each pick before any threshold or renormalisation, float64.

    softmax: p_e = exp((s_e - max s) * inv_tau) / sum_e' exp((s_e' - max s) * inv_tau)
             over all experts, evaluated at the j-th pick;
    sigmoid: 1 / (1 + exp(-s at the j-th pick)).
    Entries of ``idx`` equal to -1 give 0.
    """
    s64 = s.astype(np.float64)
    ii = np.maximum(idx.astype(np.int64), 0)
    if gate == "softmax":
        z = (s64 - s64.max(axis=1, keepdims=True)) * float(inv_temperature)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ii, axis=1)
    elif gate == "sigmoid":
        w = 1.0 / (1.0 + np.exp(-np.take_along_axis(s64, ii, axis=1)))
    else:
        raise ValueError(gate)
    return np.where(idx >= 0, w, 0.0)


def gate_weights(s: np.ndarray, idx: np.ndarray, gate: str, renorm: bool,
                 inv_temperature: float = 1.0) -> np.ndarray:
    """Gate weight of each pick, computed in float64 and stored as float32:
    the raw gate value, then, with renorm, w_j /= sum_j w_j over the picks
    that have an expert (a token whose picks were all dropped keeps zeros)."""
    w = raw_gate(s, idx, gate, inv_temperature)
    if renorm:
        tot = w.sum(axis=1, keepdims=True)
        w = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    return round_rne(w, F32).astype(np.float32)


def threshold_mask(s: np.ndarray, idx: np.ndarray, gate: str,
                   inv_temperature: float, min_prob: float) -> np.ndarray:
    """True where a pick survives the minimum-probability threshold: its raw
    gate value (float64, before renormalisation) is above min_prob (GPT-4
    MoE page, section 2.3 stage 2 and the section 4.1 sketch: picks whose
    probability is not above the minimum activation threshold are dropped).
    All True when min_prob is 0: the threshold is off."""
    if not min_prob > 0:
        return np.ones(idx.shape, dtype=bool)
    return raw_gate(s, idx, gate, inv_temperature) > float(min_prob)


def route(logits: np.ndarray, bias: Optional[np.ndarray], k: int, gate: str,
          renorm: bool, inv_temperature: float = 1.0, min_prob: float = 0.0):
    """(topk_idx int32 [T,k], topk_w float32 [T,k]) from float32 logits.

    Picks dropped by the threshold have index -1 and weight 0.  Gate values
    fall with the selection order, so the dropped picks of a token are the
    last ones.
    """
    s = selection_scores(logits, bias)
    idx = topk_select(s, k)
    keep = threshold_mask(s, idx, gate, inv_temperature, min_prob)
    idx = np.where(keep, idx, -1).astype(np.int32)
    w = gate_weights(s, idx, gate, renorm, inv_temperature)
    return idx, w


# ---------------------------------------------------------------------------
# 3. Dispatch: counts, offsets, the layout map and the permute-gather
# ---------------------------------------------------------------------------


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of (token, pick) pairs routed to expert e."""
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.reshape(-1):
        if e >= 0:          # -1: a pick dropped by the gate threshold
            counts[e] += 1
    return counts.astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e] (length E+1)."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    for e, c in enumerate(counts):
        off[e + 1] = off[e] + int(c)
    return off.astype(np.int32)


def layout_map(idx: np.ndarray, offsets: np.ndarray):
    """slot_of[t, j] and its inverse row_token[slot].

    Each expert's segment is filled in ascending token order: the j-th pick
    of token t, expert e, lands at offsets[e] + (number of earlier tokens
    that also picked e).  Dropped picks (index -1) get slot -1 and no row;
    row_token entries past offsets[E] are -1.
    """
    T, k = idx.shape
    E = len(offsets) - 1
    fill = [0] * E
    slot_of = np.full((T, k), -1, dtype=np.int32)
    row_token = np.full(T * k, -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            r = int(offsets[e]) + fill[e]
            fill[e] += 1
            slot_of[t, j] = r
            row_token[r] = t
    return slot_of, row_token


def gather_rows(x_stored: np.ndarray, row_token: np.ndarray, r_begin: int,
                r_end: int) -> np.ndarray:
    """x_perm[r] = x[row_token[r]] for r in [r_begin, r_end): a bit copy."""
    return x_stored[row_token[r_begin:r_end]]


def place_experts(idx: np.ndarray, rep_offsets: np.ndarray,
                  rep_phys: np.ndarray) -> np.ndarray:
    """Physical expert of every pick (TensorRT-LLM large-EP page, high-level
    design: routing reads the placement information of replicated experts).

    Logical expert e has copies rep_phys[rep_offsets[e]:rep_offsets[e+1]];
    pick j of token t goes to copy number t mod (number of copies).  Dropped
    picks (-1) stay -1.
    """
    T, k = idx.shape
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            b = int(rep_offsets[e])
            n = int(rep_offsets[e + 1]) - b
            out[t, j] = rep_phys[b + t % n]
    return out


def expert_load(idx: np.ndarray, E: int) -> np.ndarray:
    """Online load statistics: picks per logical expert (dropped picks not
    counted), as uint64 (the same page's GPU-side statistics component)."""
    load = np.zeros(E, dtype=np.uint64)
    for e in idx.reshape(-1):
        if e >= 0:
            load[e] += np.uint64(1)
    return load


# ---------------------------------------------------------------------------
# 4. Expert FFN
# ---------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu_erf(a: np.ndarray) -> np.ndarray:
    """Exact GELU: 0.5 * a * (1 + erf(a / sqrt(2)))."""
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def dequant_e4m3_blocks(codes: np.ndarray, scales: np.ndarray,
                        block: int = 128) -> np.ndarray:
    """W[n, c] = e4m3(code[n, c]) * scale[n // 128, c // 128], exact in float64."""
    w = e4m3_decode(codes)
    s = np.repeat(np.repeat(scales.astype(np.float64), block, axis=0), block, axis=1)
    return w * s


def expert_ffn(X: np.ndarray, w13: np.ndarray, w2: np.ndarray, act: str,
               act_dtype: str) -> np.ndarray:
    """One expert on rows X (float64 values) -> y rounded to act_dtype (float64).

    swiglu: g = X Wg^T, u = X Wu^T (Wg = w13 rows [0, I), Wu = rows [I, 2I)),
            h = rnd(silu(g) * u);
    gelu:   h = rnd(gelu_erf(X W1^T));
    then    y = rnd(h W2^T).
    """
    if act == "swiglu":
        I = w13.shape[0] // 2
        g = X @ w13[:I].T
        u = X @ w13[I:].T
        h = round_act(silu(g) * u, act_dtype)
    elif act == "gelu":
        h = round_act(gelu_erf(X @ w13.T), act_dtype)
    else:
        raise ValueError(act)
    return round_act(h @ w2.T, act_dtype)


# ---------------------------------------------------------------------------
# 5. Combine
# ---------------------------------------------------------------------------


def combine(y_perm: np.ndarray, slot_of: np.ndarray, topk_w: np.ndarray,
            act_dtype: str, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """out[t] = rnd(sum_j w[t, j] * y_perm[slot_of[t, j]]), summed in pick order
    over the picks that have a row (slot -1: dropped by the gate threshold).

    ``y_perm`` holds float64 values of the stored rows.  With ``tokens`` only
    those output rows are computed.
    """
    ts = np.arange(slot_of.shape[0]) if tokens is None else np.asarray(tokens)
    acc = np.zeros((len(ts), y_perm.shape[1]), dtype=np.float64)
    for j in range(slot_of.shape[1]):
        sj = slot_of[ts, j]
        has = sj >= 0
        if not has.any():
            continue
        acc[has] += topk_w[ts[has], j].astype(np.float64)[:, None] * y_perm[sj[has]]
    return round_act(acc, act_dtype)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------


@dataclass
class LayerParams:
    T: int
    H: int
    E: int
    k: int
    I: int
    act_dtype: str
    w_dtype: str
    gate: str
    renorm: bool
    act: str
    e_begin: int
    e_end: int
    inv_temperature: float = 1.0
    min_prob: float = 0.0
    fp8_dispatch: bool = False   # rows sent as E4M3 codes with a per-row scale


def layer_forward(p: LayerParams, x_stored: np.ndarray,
                  w_router_stored: Optional[np.ndarray],
                  bias: Optional[np.ndarray], w13_stored: np.ndarray,
                  w2_stored: np.ndarray, w13_scale: Optional[np.ndarray] = None,
                  w2_scale: Optional[np.ndarray] = None,
                  y_remote_stored: Optional[np.ndarray] = None,
                  logits: Optional[np.ndarray] = None,
                  placement=None,
                  timings: Optional[Dict[str, float]] = None) -> Dict[str, np.ndarray]:
    """The full layer on stored inputs (bit patterns / float32 values).

    ``logits`` may be given (float32) instead of being computed from the
    router weights, so that the integer steps can be re-run on exactly the
    scores another implementation produced.  Rows of experts outside
    [e_begin, e_end) are taken from ``y_remote_stored`` (outputs received
    from other GPUs); local rows are this expert FFN's results.

    ``placement`` = (rep_offsets, rep_phys, E_phys) replaces every logical
    pick by its physical copy (place_experts) before dispatch; the expert
    range and the weights are then those of the physical slots.

    ``timings``, when given, receives the wall-clock seconds of the four
    stages (route, dispatch, ffn, combine); it changes nothing computed.
    """
    clock = [time.perf_counter()]

    def lap(stage):
        if timings is not None:
            now = time.perf_counter()
            timings[stage] = timings.get(stage, 0.0) + now - clock[0]
            clock[0] = now

    x64 = decode(x_stored, p.act_dtype)
    if logits is None:
        logits = router_logits(x64, decode(w_router_stored, p.act_dtype))
    idx, w = route(logits, bias, p.k, p.gate, p.renorm, p.inv_temperature, p.min_prob)
    lap("route")
    E = p.E
    idx_log = idx
    if placement is not None:
        rep_offsets, rep_phys, E = placement
        idx = place_experts(idx, rep_offsets, rep_phys)
    counts = expert_counts(idx, E)
    offsets = expert_offsets(counts)
    slot_of, row_token = layout_map(idx, offsets)
    r0, r1 = int(offsets[p.e_begin]), int(offsets[p.e_end])
    x_perm = gather_rows(x_stored, row_token, r0, r1)
    x_scale = None
    if p.fp8_dispatch:
        # the expert FFN sees the dequantised rows: code value * row scale
        x_perm, x_scale = quantize_rows_e4m3(decode(x_perm, p.act_dtype))
        xp64 = e4m3_decode(x_perm) * x_scale.astype(np.float64)[:, None]
    else:
        xp64 = decode(x_perm, p.act_dtype)
    lap("dispatch")

    N = p.T * p.k
    if y_remote_stored is not None:
        y_perm = decode(y_remote_stored, p.act_dtype).copy()
    else:
        y_perm = np.zeros((N, p.H), dtype=np.float64)
    for el in range(p.e_end - p.e_begin):
        e = p.e_begin + el
        a, b = int(offsets[e]) - r0, int(offsets[e + 1]) - r0
        if b == a:
            continue
        w13, w2 = expert_weights(p, w13_stored, w2_stored, w13_scale, w2_scale, el)
        y_perm[r0 + a:r0 + b] = expert_ffn(xp64[a:b], w13, w2, p.act, p.act_dtype)
    lap("ffn")
    out = combine(y_perm, slot_of, w, p.act_dtype)
    lap("combine")
    return dict(logits=logits, topk_idx=idx_log, topk_phys=idx, topk_w=w, counts=counts,
                offsets=offsets, slot_of=slot_of, row_token=row_token,
                x_perm=x_perm, x_scale=x_scale, y_perm=y_perm, out=out)


def expert_weights(p: LayerParams, w13_stored, w2_stored, w13_scale, w2_scale,
                   el: int):
    """float64 weights of local expert ``el`` (decoded, dequantised)."""
    if p.w_dtype == FP8_E4M3:
        return (dequant_e4m3_blocks(w13_stored[el], w13_scale[el]),
                dequant_e4m3_blocks(w2_stored[el], w2_scale[el]))
    return decode(w13_stored[el], p.w_dtype), decode(w2_stored[el], p.w_dtype)


# ---------------------------------------------------------------------------
# Byte accounting (the pages' arithmetic)
# ---------------------------------------------------------------------------


def a2a_bytes_per_direction(counts: np.ndarray, remote_experts: Sequence[int],
                            H: int, elem_bytes: int) -> int:
    """Bytes one GPU sends for the rows routed to experts on the other GPU.

    ThunderEP page, section 1.2: with top-1 and half the tokens remote, each
    GPU sends B/2 x H x 2 bytes at dispatch, receives as many, and the same
    again at combine.
    """
    return int(sum(int(counts[e]) for e in remote_experts)) * H * elem_bytes


def expert_weight_bytes(H: int, I: int, w_bits: int, block_elems: int = 0,
                        scale_bytes: int = 0, gated: bool = True) -> int:
    """Bytes of one expert's FFN weights (plus one scale per block of values)."""
    n = (3 if gated else 2) * H * I
    b = n * w_bits // 8
    if block_elems:
        b += (n // block_elems) * scale_bytes
    return b
