"""ctypes binding of libmoe.so (the C ABI of include/moe.h).

Argument marshalling only: torch tensors are passed as device pointers and
the current HIP stream as the stream handle.  Every step of the layer runs
in the library's kernels; there is no fallback.  A missing library or a
non-zero status raises.
"""

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_TOO_LARGE = -5
NOALLOC_SCRATCH_BYTES = 1 << 20   # MOE_NOALLOC_SCRATCH_BYTES
DTYPE_F32, DTYPE_F16, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2, 3
GATE_SOFTMAX, GATE_SIGMOID = 0, 1
ACT_SWIGLU, ACT_GELU = 0, 1
WS_DISPATCH, WS_FFN, WS_FUSED = 0, 1, 2
# byte offset of moe_layer_fused's status word in its workspace (include/moe.h)
FUSED_STATUS_BYTE = 32

EXPORTS = ["moe_route", "moe_dispatch", "moe_dispatch_noalloc", "moe_dispatch_fp8", "moe_expert_ffn",
           "moe_expert_ffn_up", "moe_expert_ffn_up_fp8", "moe_expert_ffn_down",
           "moe_combine", "moe_layer_fused", "moe_place_experts", "moe_expert_load_stats",
           "moe_workspace_bytes", "moe_status_string"]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None

P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "moe_route": [P, P, I, P, I, I, I, I, I, I, F, F, P, P, P, P],
    "moe_dispatch": [P, I, P, I, I, I, I, I, I, P, P, P, P, P, P, SZ, P],
    "moe_dispatch_noalloc": [P, I, P, I, I, I, I, I, I, P, P, P, P, P, P],
    "moe_dispatch_fp8": [P, I, P, I, I, I, I, I, I, P, P, P, P, P, P, P, SZ, P],
    "moe_expert_ffn_up_fp8": [P, P, P, I, I, I, I, I, I, P, P, P, P],
    "moe_expert_ffn": [P, P, I, I, I, I, I, I, I, P, P, P, P, I, P, P, P, SZ, P],
    "moe_expert_ffn_up": [P, P, I, I, I, I, I, I, I, P, P, I, P, P, SZ, P],
    "moe_expert_ffn_down": [P, I, I, I, I, I, I, P, P, I, P, P, P, SZ, P],
    "moe_combine": [P, P, P, I, I, I, I, P, P],
    "moe_layer_fused": [P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, SZ, P],
    "moe_place_experts": [P, I, I, I, I, P, P, P, P],
    "moe_expert_load_stats": [P, I, I, I, P, P],
    "moe_workspace_bytes": [I, I, I, I, I, I],
    "moe_status_string": [I],
}


def lib() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())


DTYPE_OF = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16,
            torch.bfloat16: DTYPE_BF16, torch.uint8: DTYPE_FP8_E4M3,
            torch.float8_e4m3fn: DTYPE_FP8_E4M3}


def moe_route(x, w_router, bias, k, gate, renorm, inv_temperature, logits, topk_idx,
              topk_w, act_dtype=None, stream=None, min_prob=0.0):
    T, E = logits.shape
    H = x.shape[1] if x is not None else 0
    dt = act_dtype if act_dtype is not None else DTYPE_OF[x.dtype]
    check("moe_route", lib().moe_route(
        ptr(x), ptr(w_router), dt, ptr(bias), T, H, E, k, gate, int(renorm),
        float(inv_temperature), float(min_prob), ptr(logits), ptr(topk_idx),
        ptr(topk_w), stream_handle(stream)))


def moe_dispatch(x, topk_idx, E, e_begin, e_end, counts, offsets, slot_of, row_token,
                 x_perm, ws, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    check("moe_dispatch", lib().moe_dispatch(
        ptr(x), DTYPE_OF[x.dtype], ptr(topk_idx), T, H, E, k, e_begin, e_end,
        ptr(counts), ptr(offsets), ptr(slot_of), ptr(row_token), ptr(x_perm),
        ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_dispatch_noalloc(x, topk_idx, E, e_begin, e_end, counts, offsets, slot_of,
                         row_token, x_perm, stream=None):
    """moe_dispatch with the library's fixed scratch as its workspace."""
    T, H = x.shape
    k = topk_idx.shape[1]
    check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        ptr(x), DTYPE_OF[x.dtype], ptr(topk_idx), T, H, E, k, e_begin, e_end,
        ptr(counts), ptr(offsets), ptr(slot_of), ptr(row_token), ptr(x_perm),
        stream_handle(stream)))


def moe_dispatch_fp8(x, topk_idx, E, e_begin, e_end, counts, offsets, slot_of, row_token,
                     x_perm_q, x_scale, ws, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    check("moe_dispatch_fp8", lib().moe_dispatch_fp8(
        ptr(x), DTYPE_OF[x.dtype], ptr(topk_idx), T, H, E, k, e_begin, e_end,
        ptr(counts), ptr(offsets), ptr(slot_of), ptr(row_token), ptr(x_perm_q),
        ptr(x_scale), ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_expert_ffn_up_fp8(x_perm_q, x_scale, offsets, H, I, e_begin, e_end, max_rows, act,
                          w13, w13_scale, h_ws, stream=None):
    check("moe_expert_ffn_up_fp8", lib().moe_expert_ffn_up_fp8(
        ptr(x_perm_q), ptr(x_scale), ptr(offsets), H, I, e_begin, e_end, max_rows, act,
        ptr(w13), ptr(w13_scale), ptr(h_ws), stream_handle(stream)))


def _ws(ws):
    return (ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def moe_expert_ffn_up(x_perm, offsets, H, I, e_begin, e_end, max_rows, act, w13,
                      w13_scale, h_ws, ws=None, stream=None):
    check("moe_expert_ffn_up", lib().moe_expert_ffn_up(
        ptr(x_perm), ptr(offsets), DTYPE_OF[x_perm.dtype], H, I, e_begin, e_end,
        max_rows, act, ptr(w13), ptr(w13_scale), DTYPE_OF[w13.dtype], ptr(h_ws), *_ws(ws),
        stream_handle(stream)))


def moe_expert_ffn_down(offsets, H, I, e_begin, e_end, max_rows, w2, w2_scale, h_ws,
                        y_perm, ws=None, stream=None):
    check("moe_expert_ffn_down", lib().moe_expert_ffn_down(
        ptr(offsets), DTYPE_OF[y_perm.dtype], H, I, e_begin, e_end, max_rows, ptr(w2),
        ptr(w2_scale), DTYPE_OF[w2.dtype], ptr(h_ws), ptr(y_perm), *_ws(ws),
        stream_handle(stream)))


def moe_expert_ffn(x_perm, offsets, H, I, e_begin, e_end, max_rows, act, w13,
                   w13_scale, w2, w2_scale, h_ws, y_perm, ws=None, stream=None):
    check("moe_expert_ffn", lib().moe_expert_ffn(
        ptr(x_perm), ptr(offsets), DTYPE_OF[x_perm.dtype], H, I, e_begin, e_end,
        max_rows, act, ptr(w13), ptr(w13_scale), ptr(w2), ptr(w2_scale),
        DTYPE_OF[w13.dtype], ptr(h_ws), ptr(y_perm), *_ws(ws), stream_handle(stream)))


def moe_combine(y_perm, slot_of, topk_w, out, stream=None):
    T, H = out.shape
    k = slot_of.shape[1]
    check("moe_combine", lib().moe_combine(
        ptr(y_perm), ptr(slot_of), ptr(topk_w), DTYPE_OF[out.dtype], T, H, k, ptr(out),
        stream_handle(stream)))


def moe_layer_fused(x, offsets, slot_of, row_token, topk_w, E, I, e_begin, e_end, act,
                    w13, w2, h_ws, y_perm, out, ws, stream=None):
    T, H = x.shape
    k = slot_of.shape[1]
    check("moe_layer_fused", lib().moe_layer_fused(
        ptr(x), ptr(offsets), ptr(slot_of), ptr(row_token), ptr(topk_w),
        DTYPE_OF[x.dtype], T, H, E, k, I, e_begin, e_end, act, ptr(w13), ptr(w2),
        ptr(h_ws), ptr(y_perm), ptr(out), ptr(ws), ws.numel() * ws.element_size(),
        stream_handle(stream)))


def moe_place_experts(topk_idx, E_log, E_phys, rep_offsets, rep_phys, topk_phys,
                      stream=None):
    T, k = topk_idx.shape
    check("moe_place_experts", lib().moe_place_experts(
        ptr(topk_idx), T, k, E_log, E_phys, ptr(rep_offsets), ptr(rep_phys), ptr(topk_phys),
        stream_handle(stream)))


def moe_expert_load_stats(topk_idx, E, stats, stream=None):
    T, k = topk_idx.shape
    check("moe_expert_load_stats", lib().moe_expert_load_stats(
        ptr(topk_idx), T, k, E, ptr(stats), stream_handle(stream)))


def moe_workspace_bytes(which, T, H, E, k, I) -> int:
    return int(lib().moe_workspace_bytes(which, T, H, E, k, I))
