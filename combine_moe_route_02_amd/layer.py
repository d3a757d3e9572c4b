"""A MoE layer forward on one GPU driven through the C ABI.

Buffers are torch tensors (device memory and streams only); each step is one
call into libmoe.so: route -> dispatch -> expert FFN -> combine, or the fused
kernel after route and dispatch.  Nothing here computes any part of the
layer.
"""

import dataclasses
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L

GATES = {"softmax": L.GATE_SOFTMAX, "sigmoid": L.GATE_SIGMOID}
ACTS = {"swiglu": L.ACT_SWIGLU, "gelu": L.ACT_GELU}


@dataclass(frozen=True)
class LayerSpec:
    T: int
    H: int
    E: int
    k: int
    I: int
    act_dtype: torch.dtype
    gate: str = "softmax"
    renorm: bool = False
    act: str = "swiglu"
    e_begin: int = 0
    e_end: int = -1          # -1: all experts are local
    inv_temperature: float = 1.0
    min_prob: float = 0.0    # gate threshold; 0 = off
    fp8_dispatch: bool = False   # send dispatched rows as E4M3 codes (fp8 weights)
    E_phys: int = 0          # > 0: picks go to physical expert copies (set_placement);
                             # the local range then numbers physical slots

    @property
    def E_disp(self) -> int:
        """Experts as dispatch, the FFN and combine see them."""
        return self.E_phys if self.E_phys > 0 else self.E

    @property
    def local(self):
        return self.e_begin, (self.E_disp if self.e_end < 0 else self.e_end)

    @property
    def max_rows(self) -> int:
        e0, e1 = self.local
        return self.T * min(self.k, e1 - e0)


class MoELayer:
    """Owns the per-call buffers of one layer shape on one device."""

    def __init__(self, spec: LayerSpec, device="cuda", ffn_split=True):
        s = self.spec = spec
        dev = torch.device(device)
        N = s.T * s.k
        i32 = dict(dtype=torch.int32, device=dev)
        self.logits = torch.empty((s.T, s.E), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((s.T, s.k), **i32)
        self.topk_w = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((s.E_disp,), **i32)
        self.offsets = torch.empty((s.E_disp + 1,), **i32)
        # placement: physical expert of every pick, and its information
        self.topk_phys = torch.empty((s.T, s.k), **i32) if s.E_phys > 0 else None
        self.topk_disp = self.topk_phys if s.E_phys > 0 else self.topk_idx
        self.rep_offsets = self.rep_phys = None
        self.load_stats = None
        self.slot_of = torch.empty((s.T, s.k), **i32)
        self.row_token = torch.empty((N,), **i32)
        # fp8 transport: E4M3 codes and one scale per row instead of x_perm
        self.x_perm = torch.empty((1 if s.fp8_dispatch else N, s.H), dtype=s.act_dtype,
                                  device=dev)
        self.x_q = self.x_scale = None
        if s.fp8_dispatch:
            self.x_q = torch.empty((N, s.H), dtype=torch.uint8, device=dev)
            self.x_scale = torch.empty((max(N, 1),), dtype=torch.float32, device=dev)
        self.h = torch.empty((max(s.max_rows, 1), s.I), dtype=s.act_dtype, device=dev)
        self.y_perm = torch.zeros((N, s.H), dtype=s.act_dtype, device=dev)
        self.out = torch.empty((s.T, s.H), dtype=s.act_dtype, device=dev)
        nb = L.moe_workspace_bytes(L.WS_DISPATCH, s.T, s.H, s.E_disp, s.k, s.I)
        self.ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=dev)
        self.ws_fused = None
        # FFN workspace: lets the GEMMs split a sparse last round of tiles over
        # K; its arrival counters must start at zero (the calls keep them so)
        self.ws_ffn = None
        if ffn_split:
            nf = L.moe_workspace_bytes(L.WS_FFN, s.T, s.H, s.E_disp, s.k, s.I)
            self.ws_ffn = torch.zeros((nf,), dtype=torch.uint8, device=dev)

    # -- the four calls -----------------------------------------------------
    # -- placement hooks ------------------------------------------------------
    def set_placement(self, rep_offsets, rep_phys):
        """Copies of logical expert e: physical slots
        rep_phys[rep_offsets[e]:rep_offsets[e+1]] (int32 device tensors)."""
        assert self.spec.E_phys > 0, "the spec has no physical expert slots"
        self.rep_offsets, self.rep_phys = rep_offsets, rep_phys

    def enable_load_stats(self):
        """Accumulate picks per logical expert over route calls (int64 view of
        the uint64 counters; zero it to start a new window)."""
        self.load_stats = torch.zeros((self.spec.E,), dtype=torch.int64,
                                      device=self.out.device)

    def _after_route(self, stream):
        s = self.spec
        if self.load_stats is not None:
            L.moe_expert_load_stats(self.topk_idx, s.E, self.load_stats, stream=stream)
        if s.E_phys > 0:
            assert self.rep_offsets is not None, "set_placement() first"
            L.moe_place_experts(self.topk_idx, s.E, s.E_phys, self.rep_offsets,
                                self.rep_phys, self.topk_phys, stream=stream)

    def route(self, x, w_router, bias=None, stream=None):
        s = self.spec
        L.moe_route(x, w_router, bias, s.k, GATES[s.gate], s.renorm, s.inv_temperature,
                    self.logits, self.topk_idx, self.topk_w, stream=stream,
                    min_prob=s.min_prob)
        self._after_route(stream)

    def route_from_logits(self, bias=None, stream=None):
        """Top-k gating on the scores already in self.logits."""
        s = self.spec
        L.moe_route(None, None, bias, s.k, GATES[s.gate], s.renorm, s.inv_temperature,
                    self.logits, self.topk_idx, self.topk_w,
                    act_dtype=L.DTYPE_OF[s.act_dtype], stream=stream, min_prob=s.min_prob)
        self._after_route(stream)

    def dispatch(self, x, stream=None):
        s = self.spec
        e0, e1 = s.local
        if s.fp8_dispatch:
            L.moe_dispatch_fp8(x, self.topk_disp, s.E_disp, e0, e1, self.counts, self.offsets,
                               self.slot_of, self.row_token, self.x_q, self.x_scale,
                               self.ws, stream=stream)
            return
        L.moe_dispatch(x, self.topk_disp, s.E_disp, e0, e1, self.counts, self.offsets,
                       self.slot_of, self.row_token, self.x_perm, self.ws, stream=stream)

    def ffn_up(self, w13, w13_scale=None, stream=None):
        s = self.spec
        e0, e1 = s.local
        if s.fp8_dispatch:
            L.moe_expert_ffn_up_fp8(self.x_q, self.x_scale, self.offsets, s.H, s.I, e0, e1,
                                    s.max_rows, ACTS[s.act], w13, w13_scale, self.h,
                                    stream=stream)
            return
        L.moe_expert_ffn_up(self.x_perm, self.offsets, s.H, s.I, e0, e1, s.max_rows,
                            ACTS[s.act], w13, w13_scale, self.h, ws=self.ws_ffn,
                            stream=stream)

    def ffn_down(self, w2, w2_scale=None, stream=None):
        s = self.spec
        e0, e1 = s.local
        L.moe_expert_ffn_down(self.offsets, s.H, s.I, e0, e1, s.max_rows, w2, w2_scale,
                              self.h, self.y_perm, ws=self.ws_ffn, stream=stream)

    def ffn(self, w13, w2, w13_scale=None, w2_scale=None, stream=None):
        s = self.spec
        e0, e1 = s.local
        if s.fp8_dispatch:
            self.ffn_up(w13, w13_scale, stream)
            self.ffn_down(w2, w2_scale, stream)
            return
        L.moe_expert_ffn(self.x_perm, self.offsets, s.H, s.I, e0, e1, s.max_rows,
                         ACTS[s.act], w13, w13_scale, w2, w2_scale, self.h, self.y_perm,
                         ws=self.ws_ffn, stream=stream)

    def combine(self, stream=None):
        L.moe_combine(self.y_perm, self.slot_of, self.topk_w, self.out, stream=stream)

    def forward(self, x, w_router, bias, w13, w2, w13_scale=None, w2_scale=None,
                stream=None) -> torch.Tensor:
        self.route(x, w_router, bias, stream)
        self.dispatch(x, stream)
        self.ffn_up(w13, w13_scale, stream)
        self.ffn_down(w2, w2_scale, stream)
        self.combine(stream)
        return self.out

    # -- fused variant ------------------------------------------------------
    def fused(self, x, w13, w2, stream=None):
        s = self.spec
        e0, e1 = s.local
        if self.ws_fused is None:
            nb = L.moe_workspace_bytes(L.WS_FUSED, s.T, s.H, s.E_disp, s.k, s.I)
            self.ws_fused = torch.zeros((max(nb, 64),), dtype=torch.uint8,
                                        device=self.out.device)
        L.moe_layer_fused(x, self.offsets, self.slot_of, self.row_token, self.topk_w,
                          s.E_disp, s.I, e0, e1, ACTS[s.act], w13, w2, self.h, self.y_perm,
                          self.out, self.ws_fused, stream=stream)

    def dispatch_layout(self, x, stream=None):
        """Counts, offsets and the layout map only (no permuted copy of x):
        the fused kernel reads token rows through the layout map."""
        s = self.spec
        L.moe_dispatch(x, self.topk_disp, s.E_disp, 0, 0, self.counts, self.offsets,
                       self.slot_of, self.row_token, self.x_perm, self.ws, stream=stream)

    def fused_status(self) -> int:
        """Status word of the last completed moe_layer_fused call: 0, or 1 if a
        readiness wait timed out (out, y_perm and h may then be partly written).
        Reading it waits for the device."""
        if self.ws_fused is None:
            return 0
        return int(self.ws_fused[L.FUSED_STATUS_BYTE:L.FUSED_STATUS_BYTE + 4]
                   .view(torch.int32).item())

    def forward_fused(self, x, w_router, bias, w13, w2, stream=None) -> torch.Tensor:
        """The whole layer with the fused kernel; raises if its status word
        reports a timed-out wait."""
        self.route(x, w_router, bias, stream)
        self.dispatch_layout(x, stream)
        self.fused(x, w13, w2, stream)
        st = self.fused_status()
        if st != 0:
            raise L.MoeError("moe_layer_fused", st, "a readiness wait timed out; the "
                             "outputs are incomplete")
        return self.out


class MicrobatchedLayer:
    """The layer over token chunks on two streams (ThunderEP page, section
    3.2: micro-batches whose data movement overlaps the previous micro-batch's
    expert GEMMs; 4-8 chunks suggested).

    Each chunk is a MoELayer of its own tokens (routing is per token, so
    the chunks route exactly as the whole batch would); their outputs are
    row slices of one output tensor.  Route, dispatch and combine of every
    chunk run on the memory stream, the expert FFN on the compute stream.
    Chunk i's FFN waits for its dispatch, its combine for its FFN, and the
    memory stream takes chunk i+1's route and dispatch before chunk i's
    combine, so data movement of one chunk overlaps another chunk's GEMMs.
    Streams keep the default priority.  The FFN calls are serialised on the
    compute stream, so the chunks share one FFN workspace.
    """

    def __init__(self, spec: LayerSpec, n_chunks: int, device="cuda", ffn_split=True):
        assert 1 <= n_chunks <= max(spec.T, 1)
        dev = torch.device(device)
        self.spec = spec
        self.bounds = [spec.T * i // n_chunks for i in range(n_chunks + 1)]
        self.out = torch.empty((spec.T, spec.H), dtype=spec.act_dtype, device=dev)
        self.layers = []
        for i in range(n_chunks):
            lay = MoELayer(dataclasses.replace(spec, T=self.bounds[i + 1] - self.bounds[i]),
                           dev, ffn_split=False)
            lay.out = self.out[self.bounds[i]:self.bounds[i + 1]]
            self.layers.append(lay)
        if ffn_split:
            nf = L.moe_workspace_bytes(L.WS_FFN, spec.T, spec.H, spec.E_disp, spec.k, spec.I)
            ws = torch.zeros((nf,), dtype=torch.uint8, device=dev)
            for lay in self.layers:
                lay.ws_ffn = ws
        self.s_mem = torch.cuda.Stream(dev)
        self.s_comp = torch.cuda.Stream(dev)
        self.ev_disp = [torch.cuda.Event() for _ in range(n_chunks)]
        self.ev_ffn = [torch.cuda.Event() for _ in range(n_chunks)]

    def forward(self, x, w_router, bias, w13, w2, w13_scale=None, w2_scale=None,
                up_events=None) -> torch.Tensor:
        """up_events: optional [(start, end)] per chunk, recorded around its
        GEMM-1 on the compute stream (for timing)."""
        cur = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(cur)
        self.s_mem.wait_event(start)
        self.s_comp.wait_event(start)
        n = len(self.layers)

        def front(i):
            b0, b1 = self.bounds[i], self.bounds[i + 1]
            lay = self.layers[i]
            lay.route(x[b0:b1], w_router, bias, stream=self.s_mem)
            lay.dispatch(x[b0:b1], stream=self.s_mem)
            self.ev_disp[i].record(self.s_mem)

        front(0)
        for i in range(n):
            lay = self.layers[i]
            self.s_comp.wait_event(self.ev_disp[i])
            if up_events is not None:
                up_events[i][0].record(self.s_comp)
            lay.ffn_up(w13, w13_scale, stream=self.s_comp)
            if up_events is not None:
                up_events[i][1].record(self.s_comp)
            lay.ffn_down(w2, w2_scale, stream=self.s_comp)
            self.ev_ffn[i].record(self.s_comp)
            if i + 1 < n:
                front(i + 1)
            self.s_mem.wait_event(self.ev_ffn[i])
            lay.combine(stream=self.s_mem)
        end = torch.cuda.Event()
        end.record(self.s_mem)
        cur.wait_event(end)
        # the caller's stream now follows both streams; keep the inputs alive
        for t in (x, w_router, bias, w13, w2, w13_scale, w2_scale):
            if t is not None:
                t.record_stream(self.s_mem)
                t.record_stream(self.s_comp)
        return self.out
