"""Workload table for the MoE-layer forward: shapes, dtypes and gating flags.

Pure data, no arithmetic of the method.  The five layer shapes are:

* ``c1`` tiny fp32 layer: T=256, H=128, E=8, top-2 softmax, Linear-GELU-Linear
  expert (the plain expert form of the "GPT-4 1.8T / 2% active" page, its
  component table, and its router sketch with top-2 softmax).
* ``c2`` the ThunderEP page's byte example (section 1.2): H=4096 fp16,
  B=4096 tokens, top-1, here with an 8-expert SwiGLU FFN 4096->14336->4096.
* ``c3`` a Mixtral-8x7B-like layer (the ThunderEP page names Mixtral 8x7B in
  section 1.1): bf16, T=8192, top-2 with renormalised weights.
* ``c4`` one GPU's expert-parallel share of a DeepSeek-V3-like layer (the
  DySHARP page, section 1, names DeepSeek-V3): 256 experts, top-8 sigmoid
  gating, 32 local experts, Zipf-skewed expert popularity.
* ``c5`` the decode batch of the same expert layout with fp8 e4m3 expert
  weights and 128x128 block scales (the TensorRT-LLM large-EP page sizes
  DeepSeek-R1 experts in low precision and asks for CUDA-graph-capturable
  kernels that read sizes from device memory).
"""

from dataclasses import dataclass, field, replace
from typing import Optional

# dtype tags shared by the generator, the tests and the binding.
F32, F16, BF16, FP8_E4M3 = "f32", "f16", "bf16", "e4m3"

SOFTMAX, SIGMOID = "softmax", "sigmoid"
SWIGLU, GELU = "swiglu", "gelu"


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # routed experts (global)
    k: int            # top-k
    I: int            # expert FFN inner size
    act_dtype: str    # activation / router dtype
    w_dtype: str      # expert weight dtype (act_dtype or e4m3)
    gate: str         # softmax | sigmoid
    renorm: bool      # renormalise the k weights to sum 1
    act: str          # swiglu | gelu
    e_begin: int      # local expert range [e_begin, e_end)
    e_end: int
    seed: int
    bias: Optional[str] = None     # None | "normal" | "zipf"
    zipf_s: float = 1.2
    zipf_alpha: float = 0.0        # strength of the log-Zipf bias (c4 only)
    expert_std: Optional[float] = None   # None -> N(0,1)/sqrt(fan_in)
    remote_rows: bool = False      # pre-filled "received" rows for non-local experts
    inv_temperature: float = 1.0
    min_prob: float = 0.0          # gate threshold (0: off)
    fp8_dispatch: bool = False     # dispatched rows travel as E4M3 + per-row scale

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    @property
    def N(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


BASE_SEED = 20261203

# Zipf strength for c4.  It was found by bisection with the oracle's routing
# (tests/golden/calibrate_zipf.py) so that the busiest expert receives about
# ten times the mean load over all 256 experts on this seed's draw; the value
# is recorded in tests/golden/c4_zipf.json together with the realised ratio.
C4_ZIPF_ALPHA = 0.276

CONFIGS = {
    "c1": LayerConfig("c1", T=256, H=128, E=8, k=2, I=256, act_dtype=F32,
                      w_dtype=F32, gate=SOFTMAX, renorm=False, act=GELU,
                      e_begin=0, e_end=8, seed=BASE_SEED + 1),
    "c2": LayerConfig("c2", T=4096, H=4096, E=8, k=1, I=14336, act_dtype=F16,
                      w_dtype=F16, gate=SOFTMAX, renorm=False, act=SWIGLU,
                      e_begin=0, e_end=8, seed=BASE_SEED + 2),
    "c3": LayerConfig("c3", T=8192, H=4096, E=8, k=2, I=14336, act_dtype=BF16,
                      w_dtype=BF16, gate=SOFTMAX, renorm=True, act=SWIGLU,
                      e_begin=0, e_end=8, seed=BASE_SEED + 3, bias="normal",
                      expert_std=0.02),
    "c4": LayerConfig("c4", T=16384, H=7168, E=256, k=8, I=2048,
                      act_dtype=BF16, w_dtype=BF16, gate=SIGMOID, renorm=False,
                      act=SWIGLU, e_begin=0, e_end=32, seed=BASE_SEED + 4,
                      bias="zipf", zipf_alpha=C4_ZIPF_ALPHA, remote_rows=True),
    "c5": LayerConfig("c5", T=128, H=7168, E=256, k=8, I=2048, act_dtype=BF16,
                      w_dtype=FP8_E4M3, gate=SIGMOID, renorm=False, act=SWIGLU,
                      e_begin=0, e_end=32, seed=BASE_SEED + 5, remote_rows=True),
}

# Generator stream ids, one per tensor kind.
STREAM_X, STREAM_WR, STREAM_BIAS, STREAM_W13, STREAM_W2, STREAM_REMOTE, \
    STREAM_ZIPF_PERM = 1, 2, 3, 4, 5, 6, 7
