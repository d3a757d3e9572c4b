"""MI355X-native MoE expert-parallel layer forward (one GPU's share).

route -> dispatch -> grouped expert FFN -> combine, as hand-written HIP
kernels for gfx950 behind the C ABI of include/moe.h (libmoe.so).
"""

from ._lib import (MoeError, lib, moe_combine, moe_dispatch, moe_dispatch_fp8,  # noqa: F401
                   moe_expert_ffn, moe_expert_ffn_down, moe_expert_ffn_up,
                   moe_expert_ffn_up_fp8, moe_expert_load_stats, moe_layer_fused,
                   moe_place_experts, moe_route, moe_workspace_bytes)
from .layer import LayerSpec, MicrobatchedLayer, MoELayer  # noqa: F401
