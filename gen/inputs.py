"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the CPU oracle and the HIP path; it only produces
input bytes and holds none of the layer's arithmetic.

Random numbers come from a counter-based SplitMix64 stream (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
output function is the one in Vigna's public-domain splitmix64.c):

    key(seed, stream) = mix64(seed * GOLDEN + stream)
    u64(i)            = mix64(key + (i + 1) * GOLDEN)          (mod 2**64)
    mix64(z)          = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
                        z ^= z >> 27; z *= 0x94D049BB133111EB; z ^ (z >> 31)

so element i of a stream does not depend on how the tensor is chunked or on
the device.  A uniform in (0, 1] is ((u64 >> 11) + 1) * 2**-53 and a standard
normal uses Box-Muller on the pair (2i, 2i+1):
n_i = sqrt(-2 ln u(2i)) * cos(2 pi u(2i+1)), evaluated in float64.

Normals are scaled in float64, rounded to float32 (RNE), then to the target
dtype (RNE).  Both sides always consume the same stored bytes, so the
transcendental functions used here never need to agree across devices.
"""

import math
from typing import Dict, Optional

import torch

from .configs import (BF16, F16, F32, FP8_E4M3, STREAM_BIAS, STREAM_REMOTE,
                      STREAM_W13, STREAM_W2, STREAM_WR, STREAM_X,
                      STREAM_ZIPF_PERM, SWIGLU, LayerConfig)

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}

_CHUNK = 1 << 24  # elements per generation chunk (bounds temporary memory)


def _s64(v: int) -> int:
    """Python int in [0, 2**64) -> the int64 with the same bits."""
    v &= M64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference form)."""
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return mix64_int((seed * GOLDEN + stream) & M64)


def u64_int(seed: int, stream: int, i: int) -> int:
    """Element i of a stream, computed with Python integers."""
    return mix64_int(stream_key(seed, stream) + (i + 1) * GOLDEN)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return torch.bitwise_and(torch.bitwise_right_shift(z, s), (1 << (64 - s)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = torch.bitwise_xor(z, _lsr(z, 30)) * _s64(MIX1)
    z = torch.bitwise_xor(z, _lsr(z, 27)) * _s64(MIX2)
    return torch.bitwise_xor(z, _lsr(z, 31))


def u64_tensor(seed: int, stream: int, start: int, n: int,
               device="cpu") -> torch.Tensor:
    """Elements [start, start+n) of a stream as int64 bit patterns."""
    key = _s64(stream_key(seed, stream))
    ctr = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64_t(ctr * _s64(GOLDEN) + key)


def uniform_tensor(seed, stream, start, n, device="cpu") -> torch.Tensor:
    """Uniforms in (0, 1] as float64, elements [start, start+n)."""
    v = _lsr(u64_tensor(seed, stream, start, n, device), 11)
    return (v.to(torch.float64) + 1.0) * (2.0 ** -53)


def normal_tensor(seed, stream, start, n, device="cpu") -> torch.Tensor:
    """Standard normals (float64), elements [start, start+n) of the stream."""
    u = uniform_tensor(seed, stream, 2 * start, 2 * n, device).view(n, 2)
    return torch.sqrt(-2.0 * torch.log(u[:, 0])) * torch.cos((2.0 * math.pi) * u[:, 1])


def fill_normal(out: torch.Tensor, seed: int, stream: int, std: float = 1.0,
                offset: int = 0) -> torch.Tensor:
    """Fill ``out`` (contiguous, any float dtype) with std * N(0,1).

    Element j of ``out`` takes normal number ``offset + j`` of the stream.
    """
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        v = normal_tensor(seed, stream, offset + s, m, out.device) * std
        flat[s:s + m] = v.to(torch.float32).to(out.dtype)
    return out


def normal(shape, dtype, seed, stream, std=1.0, device="cpu") -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=device)
    return fill_normal(t, seed, stream, std)


# ---------------------------------------------------------------------------
# fp8 e4m3 (OCP E4M3FN) block-quantised expert weights
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def quantize_e4m3_blocks(w32: torch.Tensor, block: int = 128):
    """[G, R, C] float32 -> (codes uint8 [G, R, C], scales f32 [G, R/b, C/b]).

    Per 128x128 tile: scale = amax / 448 and code = RNE(w / scale) clamped to
    the finite range (torch's float8_e4m3fn cast rounds to nearest even).
    This is input preparation; the weights that both sides use are the codes
    and scales it returns.
    """
    G, R, C = w32.shape
    assert R % block == 0 and C % block == 0
    tiles = w32.view(G, R // block, block, C // block, block)
    amax = tiles.abs().amax(dim=(2, 4))                       # [G, R/b, C/b]
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = tiles / scale[:, :, None, :, None]
    q = q.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).reshape(G, R, C).contiguous()
    return codes, scale.to(torch.float32).contiguous()


# ---------------------------------------------------------------------------
# Layer inputs
# ---------------------------------------------------------------------------


def zipf_bias(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    """Per-expert log-Zipf selection bias: -s * alpha * ln(rank_e).

    Expert ``e_begin`` (a local expert) is rank 1; the other experts receive
    ranks 2..E in the order of a seeded random permutation.
    """
    E = cfg.E
    u = uniform_tensor(cfg.seed, STREAM_ZIPF_PERM, 0, E, "cpu")
    others = [e for e in range(E) if e != cfg.e_begin]
    order = sorted(others, key=lambda e: (float(u[e]), e))
    rank = [0] * E
    rank[cfg.e_begin] = 1
    for r, e in enumerate(order):
        rank[e] = r + 2
    b = torch.tensor([-cfg.zipf_s * cfg.zipf_alpha * math.log(r) for r in rank],
                     dtype=torch.float64)
    return b.to(torch.float32).to(device)


def make_inputs(cfg: LayerConfig, device="cpu",
                with_weights: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """All input tensors of one layer invocation, generated on ``device``.

    Keys: x [T,H], w_router [E,H], bias [E] or None, w13 [E_loc, 2I|I, H],
    w2 [E_loc, H, I], w13_scale / w2_scale (fp8 only), y_remote [T*k, H] or
    None (pre-filled rows standing in for outputs received from other GPUs).
    """
    act = TORCH_DTYPE[cfg.act_dtype]
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal((T, H), act, cfg.seed, STREAM_X, 1.0, device)
    out["w_router"] = normal((E, H), act, cfg.seed, STREAM_WR,
                             1.0 / math.sqrt(H), device)
    if cfg.bias == "normal":
        out["bias"] = normal((E,), torch.float32, cfg.seed, STREAM_BIAS, 1.0, device)
    elif cfg.bias == "zipf":
        out["bias"] = zipf_bias(cfg, device)
    else:
        out["bias"] = None

    out["w13"] = out["w2"] = out["w13_scale"] = out["w2_scale"] = None
    if with_weights:
        rows1 = 2 * I if cfg.act == SWIGLU else I
        std1 = cfg.expert_std if cfg.expert_std is not None else 1.0 / math.sqrt(H)
        std2 = cfg.expert_std if cfg.expert_std is not None else 1.0 / math.sqrt(I)
        if cfg.w_dtype == FP8_E4M3:
            w13 = normal((cfg.E_loc, rows1, H), torch.float32, cfg.seed, STREAM_W13,
                         std1, device)
            out["w13"], out["w13_scale"] = quantize_e4m3_blocks(w13)
            del w13
            w2 = normal((cfg.E_loc, H, I), torch.float32, cfg.seed, STREAM_W2,
                        std2, device)
            out["w2"], out["w2_scale"] = quantize_e4m3_blocks(w2)
            del w2
        else:
            wdt = TORCH_DTYPE[cfg.w_dtype]
            out["w13"] = normal((cfg.E_loc, rows1, H), wdt, cfg.seed, STREAM_W13,
                                std1, device)
            out["w2"] = normal((cfg.E_loc, H, I), wdt, cfg.seed, STREAM_W2, std2,
                               device)
    out["y_remote"] = (normal((cfg.N, H), act, cfg.seed, STREAM_REMOTE, 1.0, device)
                       if cfg.remote_rows else None)
    return out
