"""Benchmark of the MoE-layer forward on one MI355X.

One step = route -> dispatch -> expert FFN (GEMM-1 + SwiGLU, GEMM-2) ->
combine over one batch of synthetic tokens, every step through the C ABI of
libmoe.so on one HIP stream, inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--config c4] [--gpus 1]
                    [--fused] [--graph on|off|auto] [--flush on|off|auto]
                    [--temperature T] [--min-prob P] [--fp8-dispatch]

Defaults: the DeepSeek-V3-like EP share (c4, the largest single-GPU layer),
10 warm-up steps, then 50 timed steps, each bracketed by its own HIP events;
the line reports their median.  The decode layer (c5) is timed as replays of
one captured hipGraph, and the tiny layer (c1) reads a 512 MiB buffer
between steps so that its inputs come from HBM, not the MALL.  The flush
reads rather than writes: a written buffer leaves the MALL full of dirty
lines whose write-back then competes with the next step's reads.  The
decode layer needs none: each step streams 1.4 GB of expert weights, 5.5
times the MALL, in the same order, so nothing survives to the next step.

Prints one JSON line: whole-layer tokens/s, plus the dominant kernel's
roofline (GEMM-1, timed live with HIP events on the launch stream), the
dispatch+combine HBM rate and grouped-GEMM MFMA utilisation, and the CPU
oracle timed per stage on a bounded sample of the same workload.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0        # dense bf16 / fp16 MFMA
METRIC = "MoE-layer tokens/sec on 1 GPU; dispatch+combine HBM GB/s; GEMM MFMA % of peak"
WORKLOAD = {
    "c1": "tiny fp32 layer: T=256, H=128, E=8, top-2 softmax, GELU FFN 128->256->128",
    "c2": "ThunderEP section 1.2 shape, fp16: T=4096, H=4096, E=8, top-1 softmax, "
          "SwiGLU FFN 4096->14336->4096",
    "c3": "Mixtral-8x7B-like, bf16: T=8192, H=4096, E=8, top-2 renormalised softmax "
          "with per-expert bias, SwiGLU 4096->14336->4096",
    "c4": "DeepSeek-V3-like EP share, bf16: T=16384, H=7168, 256 experts (32 local), "
          "top-8 sigmoid, Zipf load, SwiGLU 7168->2048->7168",
    "c5": "decode batch, bf16 activations, fp8 e4m3 experts: T=128, H=7168, 256 experts "
          "(32 local), top-8 sigmoid, SwiGLU 7168->2048->7168",
}
DT_NAME = {"f32": "f32", "f16": "f16", "bf16": "bf16"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 10; 200 replays when the step "
                         "is timed as hipGraph replays, whose launch path takes a few "
                         "hundred replays to reach its steady state)")
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOAD),
                    help="workload (default c4, the largest single-GPU layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the "
                         "steps (the reference for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="turn two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calib-copy-mib run into the per-launch HBM traffic summary")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="turn a rocprofv3 --kernel-trace --stats CSV into a text summary")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PMC_CSV", "OUT"),
                    help="turn a rocprofv3 --pmc CSV (any SQ/GRBM counters) into "
                         "per-kernel medians per dispatch, with MFMA busy and wait "
                         "fractions when their counters are present")
    ap.add_argument("--dense-gemm", action="store_true",
                    help="time the library's GEMM (moe_expert_ffn_down, one expert) "
                         "and hipBLASLt (torch.matmul) on the dense bf16 product "
                         "4096 x 28672 x 4096, and print one JSON line")
    ap.add_argument("--fused", action="store_true",
                    help="time the fused dispatch->GEMM->combine kernel instead of "
                         "the four separate calls")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="softmax temperature of the gate (default: the workload's, 1.0)")
    ap.add_argument("--min-prob", type=float, default=0.0,
                    help="minimum-probability threshold of the gate (0: off)")
    ap.add_argument("--replicate-hot", type=int, default=0, metavar="R",
                    help="give the most loaded local expert R extra physical copies "
                         "(placement hook) and collect per-expert load statistics")
    ap.add_argument("--microbatch", type=int, default=0, metavar="N",
                    help="run the layer as N token chunks on two streams (data movement "
                         "of one chunk overlapping another's expert GEMMs)")
    ap.add_argument("--graph", choices=["on", "off", "auto"], default="auto",
                    help="time replays of the whole step captured in one hipGraph "
                         "(per-stage times then come from one graph per stage); "
                         "auto: on for the decode layer c5, whose workload is one "
                         "captured graph")
    ap.add_argument("--flush", choices=["on", "off", "auto"], default="auto",
                    help="read a 512 MiB buffer between timed steps (outside each "
                         "step's events) so that inputs do not stay in the 256 MiB "
                         "MALL; auto: on for the tiny layer c1 (the decode layer's own "
                         "1.4 GB weight stream evicts everything between its steps)")
    ap.add_argument("--fp8-dispatch", action="store_true",
                    help="send the dispatched rows as E4M3 codes with a per-row scale "
                         "into an fp8 x fp8 GEMM-1 (fp8-weight workloads)")
    return ap.parse_args()


def gating_of(args):
    """Workload overrides for the gating variants, and their label."""
    kw, tag = {}, []
    if args.temperature > 0:
        kw["inv_temperature"] = 1.0 / args.temperature
        tag.append(f"temperature {args.temperature:g}")
    if args.min_prob > 0:
        kw["min_prob"] = args.min_prob
        tag.append(f"threshold {args.min_prob:g}")
    label = (" [gate " + ", ".join(tag) + "]") if tag else ""
    if args.fp8_dispatch:
        kw["fp8_dispatch"] = True
        label += " [fp8 dispatch transport]"
    return kw, label


# Sources that define each measured kernel: a counter summary is valid for
# the kernel as long as these files are unchanged.
KERNEL_SOURCES = {
    "gemm1": ["gemm.hip", "gemm_tile.h", "moe_internal.h", "moe_common.h"],
    "fused": ["fused.hip", "gemm_tile.h", "moe_internal.h", "moe_common.h"],
}


def source_hash(kernel_key: str = "") -> str:
    """Hash of the kernel's defining sources (all of csrc/ without a key)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_moe_route_02_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel_key) or sorted(os.listdir(csrc))
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_hash") != source_hash(kernel_key):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary, calib_mib=args.calib_copy_mib or 1024,
                           workload=args.config, extra="--fused" if args.fused else "")
    if args.counter_summary:
        return counter_summary(*args.counter_summary, workload=args.config,
                               dense=args.dense_gemm, extra="--fused" if args.fused else "")
    if args.dense_gemm:
        return dense_gemm(args)
    if args.stats_summary:
        return stats_summary(*args.stats_summary, workload=args.config,
                             extra="--fused" if args.fused else "")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this "
              "build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from gen.configs import CONFIGS
    from gen.inputs import make_inputs
    from combine_moe_route_02_amd import LayerSpec, MoELayer
    from combine_moe_route_02_amd._lib import lib

    lib()  # fail loudly if the HIP library is missing
    gate_kw, gate_tag = gating_of(args)
    cfg = CONFIGS[args.config].with_(**gate_kw)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} inputs on {dev}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg, dev)
    tdt = inp["x"].dtype
    spec = LayerSpec(T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k, I=cfg.I, act_dtype=tdt,
                     gate=cfg.gate, renorm=cfg.renorm, act=cfg.act, e_begin=cfg.e_begin,
                     e_end=cfg.e_end, inv_temperature=cfg.inv_temperature,
                     min_prob=cfg.min_prob, fp8_dispatch=cfg.fp8_dispatch)
    if cfg.fp8_dispatch and (cfg.w_dtype != "e4m3" or args.fused):
        sys.exit("--fp8-dispatch needs an fp8-weight workload (c5) and the unfused path")
    lay = MoELayer(spec, dev)
    x, wr, bias = inp["x"], inp["w_router"], inp["bias"]
    w13, w2, s13, s2 = inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"]
    R = args.replicate_hot
    if R > 0:
        if args.fused or cfg.w_dtype == "e4m3":
            sys.exit("--replicate-hot runs the unfused 16-bit-weight path")
        # the most loaded local expert (from one routing pass, untimed) gets R
        # copies at physical slots e_end .. e_end+R-1; experts above the local
        # range move up by R
        lay.route(x, wr, bias)
        e0, e1 = cfg.e_begin, cfg.e_end
        picks = lay.topk_idx.flatten()
        cnt = torch.bincount(picks[picks >= 0].long(), minlength=cfg.E)
        hot = e0 + int(cnt[e0:e1].argmax())
        phys_of = [e if e < e1 else e + R for e in range(cfg.E)]
        rep_off = [0]
        rep_phys = []
        for e in range(cfg.E):
            rep_phys.append(phys_of[e])
            if e == hot:
                rep_phys += list(range(e1, e1 + R))
            rep_off.append(len(rep_phys))
        spec = dataclasses.replace(spec, E_phys=cfg.E + R, e_end=e1 + R)
        del lay
        lay = MoELayer(spec, dev)
        lay.set_placement(torch.tensor(rep_off, dtype=torch.int32, device=dev),
                          torch.tensor(rep_phys, dtype=torch.int32, device=dev))
        lay.enable_load_stats()
        loc = torch.arange(e0, e1, device=dev)
        own = torch.cat([loc - e0, torch.full((R,), hot - e0, device=dev, dtype=loc.dtype)])
        w13, w2 = w13[own].contiguous(), w2[own].contiguous()
        gate_tag += f" [expert {hot} replicated {R}x, load statistics on]"
    if inp["y_remote"] is not None:
        lay.y_perm.copy_(inp["y_remote"])
    stream = torch.cuda.current_stream()
    NB = args.microbatch
    if NB > 1:
        if args.fused or R > 0:
            sys.exit("--microbatch runs the unfused layer without placement")
        from combine_moe_route_02_amd import MicrobatchedLayer
        mb = MicrobatchedLayer(spec, NB, dev)
        if inp["y_remote"] is not None:     # received rows: each chunk's own slice
            for c in mb.layers:
                c.y_perm.copy_(inp["y_remote"][: c.y_perm.shape[0]])
        gate_tag += f" [{NB} micro-batches on two streams]"
        up_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(NB)] for _ in range(args.steps)]

    def step(ev=None, i=None):
        if NB > 1:
            mb.forward(x, wr, bias, w13, w2, s13, s2,
                       up_events=up_ev[i] if i is not None else None)
            return
        lay.route(x, wr, bias)
        if args.fused:
            lay.dispatch_layout(x)
        else:
            lay.dispatch(x)
        if ev is not None:
            ev[0].record(stream)
        if args.fused:
            lay.fused(x, w13, w2)
            if ev is not None:
                ev[1].record(stream)
            return
        lay.ffn_up(w13, s13)
        if ev is not None:
            ev[1].record(stream)
        lay.ffn_down(w2, s2)
        lay.combine()

    use_graph = args.graph == "on" or (args.graph == "auto" and cfg.name == "c5"
                                       and NB <= 1 and not args.fused and R == 0)
    # c1 fits in the MALL whole; the decode layer (c5) streams 1.4 GB of expert
    # weights per step, 5.5x the MALL, so nothing a step reads is still there
    # when the next one starts and a flush would only add its own write-back
    flush = args.flush == "on" or (args.flush == "auto" and cfg.name == "c1")
    flush_buf = (torch.ones(64 << 20, dtype=torch.int64, device=dev) if flush else None)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)      # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del a, b
    if use_graph and (NB > 1 or args.fused):
        sys.exit("--graph captures the unfused single-stream step")
    if args.warmup is None:
        # measured on the decode layer: 0.274 ms per replay after 10 warm-up
        # replays, 0.263 after 50-500, 0.255 after 1000 (eager: 0.254)
        args.warmup = 200 if use_graph else 10
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    graph = None
    if use_graph:
        # warm up on a side stream, then capture one whole step; every size
        # the step needs is read on the device, so replays are complete steps
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(min(max(args.warmup, 1), 10)):
                step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        # the warm-up steps of a graph run are replays of the graph
        for _ in range(max(args.warmup, 1)):
            graph.replay()
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # -- timed region: exactly K steps ------------------------------------
    # Each step is bracketed by its own pair of events on the launch stream;
    # ms_per_step is their median.  With the MALL flush on, the flush runs
    # between a step's end event and the next step's start event.
    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(K):
        if flush_buf is not None:
            flush_sum = flush_buf.sum()  # reads all 512 MiB, writes nothing large
        sev[i][0].record(stream)
        if graph is not None:
            graph.replay()
        else:
            step(kev[i], i)
        sev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([a.elapsed_time(b) for a, b in sev])
    ms_per_step = float(np.median(step_ms))
    bracket_ms = t0.elapsed_time(t1) / K
    if graph is not None:
        # GEMM-1 launches on the same stream, eager, between events (each
        # launch is long against the host's launch overhead)
        for a, b in kev:
            a.record(stream)
            lay.ffn_up(w13, s13)
            b.record(stream)
        torch.cuda.synchronize()
    if NB > 1:   # GEMM-1 launches of every chunk, on the compute stream
        g1 = np.array([a.elapsed_time(b) for st in up_ev for a, b in st])
    else:
        g1 = np.array([a.elapsed_time(b) for a, b in kev])
    gemm1_ms = float(np.mean(g1))
    print(f"[bench] {K} steps: median {ms_per_step:.4f} ms/step, mean of the bracket "
          f"{bracket_ms:.4f} ms (wall {wall:.3f} s)", file=sys.stderr, flush=True)

    # -- per-stage times (outside the timed region) ------------------------
    names = ["route", "dispatch", "ffn_up", "ffn_down", "combine"]
    calls = [lambda: lay.route(x, wr, bias), lambda: lay.dispatch(x),
             lambda: lay.ffn_up(w13, s13), lambda: lay.ffn_down(w2, s2),
             lambda: lay.combine()]
    reps = max(3, min(K, 10))
    if graph is not None:
        # one graph per stage, replayed back to back: the stage's own kernel
        # time, without the host's launch gaps between short kernels
        stage_ms = {}
        for n, c in zip(names, calls):
            gs = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs):
                c()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(50):   # replays reach their steady state after warm-up
                gs.replay()
            a.record(stream)
            for _ in range(reps):
                gs.replay()
            b.record(stream)
            torch.cuda.synchronize()
            stage_ms[n] = a.elapsed_time(b) / reps
            del gs
    else:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(reps)]
        for r in range(reps):
            ev[r][0].record(stream)
            for j, c in enumerate(calls):
                c()
                ev[r][j + 1].record(stream)
        torch.cuda.synchronize()
        stage_ms = {n: float(np.median([ev[r][j].elapsed_time(ev[r][j + 1])
                                        for r in range(reps)])) for j, n in enumerate(names)}

    # -- algorithmic bytes and flops from this run's counts ---------------
    counts = lay.counts.cpu().numpy().astype(np.int64)
    idx = lay.topk_disp.cpu().numpy()      # physical slots when experts are placed
    e0, e1 = lay.spec.local
    rows_loc = int(counts[e0:e1].sum())
    ab = x.element_size()
    H, I, T, k, E = cfg.H, cfg.I, cfg.T, cfg.k, cfg.E
    loc_pick = (idx >= e0) & (idx < e1)
    tok_needed = int(loc_pick.any(axis=1).sum())
    row_out = (H + 4) if cfg.fp8_dispatch else H * ab              # codes + scale
    disp_bytes = (tok_needed * H * ab + rows_loc * row_out         # gather
                  + T * k * 4 * 3 + E * 4 * 2)                    # idx in, slot/row out
    n_kept = int((idx >= 0).sum())                                # picks with a row
    comb_bytes = n_kept * H * ab + T * H * ab + T * k * 8         # rows in, out, slot+w
    dc_gbps = (disp_bytes + comb_bytes) / ((stage_ms["dispatch"] + stage_ms["combine"]) * 1e6)
    touched = int((counts[e0:e1] > 0).sum())
    if cfg.w_dtype == "e4m3":
        wb1 = touched * 2 * I * H * 1 + touched * (2 * I // 128) * (H // 128) * 4
    else:
        wb1 = touched * 2 * I * H * w13.element_size()
    flops1 = 2.0 * rows_loc * H * 2 * I
    flops2 = 2.0 * rows_loc * I * H
    gemm_tflops = (flops1 + flops2) / ((stage_ms["ffn_up"] + stage_ms["ffn_down"]) * 1e9)
    # layer roofline: each stage at the larger of its bytes over 8 TB/s and its
    # flops over the 16-bit matrix peak, summed over the stages
    wbytes = wb1 + (touched * H * I * (1 if cfg.w_dtype == "e4m3" else w13.element_size()))
    route_bytes = T * H * ab + E * H * ab + T * E * 4 * 2 + T * k * 8
    ffn_bytes = wbytes + rows_loc * (H * ab + 2 * I * ab + H * ab)
    stage_roof_ms = {
        "route": max(route_bytes / (PEAK_HBM_GBPS * 1e6), 2.0 * T * H * E / (PEAK_MFMA_TFLOPS * 1e9)),
        "dispatch": disp_bytes / (PEAK_HBM_GBPS * 1e6),
        "ffn": max(ffn_bytes / (PEAK_HBM_GBPS * 1e6), (flops1 + flops2) / (PEAK_MFMA_TFLOPS * 1e9)),
        "combine": comb_bytes / (PEAK_HBM_GBPS * 1e6),
    }
    layer_roof_ms = sum(stage_roof_ms.values())
    if args.fused:
        flops1 += flops2   # the fused kernel runs both GEMMs (and combine)
    if NB > 1:
        flops1 /= NB       # one GEMM-1 launch per micro-batch (average share)
        wb1_share = 1.0 / NB
    else:
        wb1_share = 1.0
    if cfg.w_dtype == "e4m3":
        bytes1 = wb1 + (rows_loc * row_out + rows_loc * I * ab) * wb1_share
        achieved = bytes1 / (gemm1_ms * 1e6)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "algorithmic_bytes_per_launch": int(bytes1)}
    else:
        achieved = flops1 / (gemm1_ms * 1e9)
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                "algorithmic_flops_per_launch": int(flops1)}
    n_loc = max(1, e1 - e0)
    if args.fused:
        kname = "fused_layer_kernel (GEMM-1 + SwiGLU + GEMM-2 + combine, moe_layer_fused)"
    elif cfg.fp8_dispatch:
        kname = "grouped_gemm_fp8s (GEMM-1 + SwiGLU, fp8 activations x fp8 weights, " \
                "moe_expert_ffn_up_fp8)"
    elif cfg.w_dtype == "e4m3":
        small_m = lay.spec.max_rows / n_loc <= 48
        kname = ("grouped_gemm_fp8s" if small_m else "grouped_gemm_mfma") + \
            " (GEMM-1 + SwiGLU, fp8 weights, moe_expert_ffn_up)"
    elif cfg.act_dtype == "f32":
        kname = f"grouped_gemm_f32 (GEMM-1 + {cfg.act.upper()}, moe_expert_ffn_up)"
    else:
        kname = f"grouped_gemm_dma (GEMM-1 + {'SwiGLU' if cfg.act == 'swiglu' else 'GELU'}, " \
                "moe_expert_ffn_up)"
    if NB > 1:
        kname += f", one launch per micro-batch of {T // NB} tokens"
    roof["kernel"] = kname
    roof["avg_launch_ms"] = round(gemm1_ms, 5)
    roof["median_launch_ms"] = round(float(np.median(g1)), 5)
    roof["launches_timed"] = int(len(g1))
    # counters were taken on the workload's own gating only
    roof["traffic"] = None if gate_tag else load_traffic("fused" if args.fused else "gemm1",
                                                         cfg.name)

    res = {
        "metric": METRIC,
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "timing": {"per_step": "median of per-step HIP events on the launch stream",
                   "mean_ms_per_step": round(float(np.mean(step_ms)), 5),
                   "min_ms_per_step": round(float(np.min(step_ms)), 5),
                   "bracket_ms_per_step": round(bracket_ms, 5),
                   "mall_flush_between_steps": bool(flush_buf is not None),
                   "mall_flush": "read of 512 MiB" if flush_buf is not None else None,
                   "graph_replay": graph is not None},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DT_NAME[cfg.act_dtype] + ("+e4m3w" if cfg.w_dtype == "e4m3" else "")
        + ("+e4m3a" if cfg.fp8_dispatch else ""),
        "data": "synthetic (seeded generator; random-init weights)",
        "config": {"workload": f"{cfg.name}: {WORKLOAD[cfg.name]}"
                   + (" [fused kernel]" if args.fused else "") + gate_tag
                   + (" [one hipGraph per step]" if graph is not None else ""), "tokens": T,
                   "hidden": H, "experts": E, "local_experts": e1 - e0, "top_k": k,
                   "ffn_inner": I, "local_rows": rows_loc, "kept_picks": n_kept},
        "roofline": roof,
        "stages_ms": {n: round(v, 5) for n, v in stage_ms.items()},
        "dispatch_combine_GBps": round(dc_gbps, 1),
        "dispatch_combine_frac_hbm": round(dc_gbps / PEAK_HBM_GBPS, 4),
        "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_mfma": round(gemm_tflops / PEAK_MFMA_TFLOPS, 4),
        "layer_roofline": {"ms": round(layer_roof_ms, 5),
                           "tokens_per_s": round(T / layer_roof_ms * 1e3, 1),
                           "frac": round(layer_roof_ms / ms_per_step, 4),
                           "stages_ms": {n: round(v, 5) for n, v in stage_roof_ms.items()}},
        "tokens_per_s_without_route": round(T / max(ms_per_step - stage_ms["route"], 1e-9) * 1e3, 1),
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_kernel(rows, counter):
    """{kernel name: [value per dispatch]} for one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_csv, write_csv, out_path, calib_mib, workload, extra=""):
    """HBM traffic per GEMM-1 launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the plain
    copy of calib_mib MiB (true bytes: calib_mib MiB read and written)."""
    import numpy as np
    fetch = _per_kernel(_counter_rows(fetch_csv), "FETCH_SIZE")
    write = _per_kernel(_counter_rows(write_csv), "WRITE_SIZE")
    # the calibration copy is the runtime's buffer copy of calib_mib MiB
    # (b.copy_(a) on contiguous uint8 tensors).  Input generation copies too,
    # some of them larger, so it is found by its WRITE_SIZE (exact for a
    # copy: calib_mib MiB) and its FETCH_SIZE taken from the copy at the same
    # position of the other run (both runs launch the same sequence).
    true_kib = calib_mib * 1024.0

    def copies(path, counter):
        rows = [r for r in _counter_rows(path)
                if r["Counter_Name"] == counter and r["Kernel_Name"] == "__amd_rocclr_copyBuffer"]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [float(r["Counter_Value"]) for r in rows]
    cw_all = copies(write_csv, "WRITE_SIZE")
    cf_all = copies(fetch_csv, "FETCH_SIZE")
    if not cw_all or len(cw_all) != len(cf_all):
        raise SystemExit("calibration copy not found in the counter CSVs")
    i = min(range(len(cw_all)), key=lambda j: abs(cw_all[j] - true_kib))
    if abs(cw_all[i] - true_kib) > 0.01 * true_kib:
        raise SystemExit("no copy of the calibration size in the WRITE_SIZE run")
    cf, cw = cf_all[i], cw_all[i]
    f_scale, w_scale = true_kib / cf, true_kib / cw
    def is_gemm1(name):
        if "fused_layer" in name:
            return True
        if "grouped_gemm" not in name or "<" not in name:
            return False
        targs = [a.strip() for a in name.split("<", 1)[1].split(">", 1)[0].split(",")]
        epi = targs[2] if "grouped_gemm_mfma" in name else targs[1]  # SwiGLU epilogue = 1
        return epi == "1"
    gemm = [k for k in fetch if is_gemm1(k)]
    what = ("the fused layer kernel (GEMM-1 + SwiGLU + GEMM-2 + combine)" if extra
            else "the GEMM-1 (+SwiGLU) kernel")
    lines = [f"# HBM traffic per launch of {what}, workload {workload}",
             "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs,",
             f"# each scaled by the same counter's reading for a plain {calib_mib} MiB copy",
             f"# copy kernel: FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB "
             f"(true {true_kib:.0f} KiB each) -> scales {f_scale:.4f}, {w_scale:.4f}",
             "# commands (from /tmp, TMPDIR=/tmp, R = repository root):",
             f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <dir_f> -o pmc -- python3 $R/bench.py "
             f"--config {workload} --steps 3 --warmup 1 --no-cpu-baseline --calib-copy-mib {calib_mib} {extra}".rstrip(),
             f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <dir_w> -o pmc -- python3 $R/bench.py "
             f"--config {workload} --steps 3 --warmup 1 --no-cpu-baseline --calib-copy-mib {calib_mib} {extra}".rstrip(),
             f"#   python3 $R/bench.py --config {workload} --calib-copy-mib {calib_mib} {extra} ".replace("  ", " ") +
             "--pmc-summary <dir_f>/pmc_counter_collection.csv <dir_w>/pmc_counter_collection.csv <out>"]
    rec = {}
    for k in gemm:
        fk = float(np.median(fetch[k]))
        wk = float(np.median(write.get(k, [0.0])))
        hbm = (fk * f_scale + wk * w_scale) * 1024.0
        lines.append(f"# kernel {k[:110]}: dispatches {len(fetch[k])}, "
                     f"FETCH_SIZE {fk:.0f} KiB, WRITE_SIZE {wk:.0f} KiB, HBM {hbm / 1e6:.1f} MB")
        rec.setdefault("hbm_bytes_per_launch", hbm)
        rec.setdefault("fetch_kib_per_launch", fk)
        rec.setdefault("write_kib_per_launch", wk)
    # every kernel of the library, for the HBM rates of route, dispatch and
    # combine (divide by the kernel-trace medians of the same workload)
    lines.append("# every library kernel: median FETCH_SIZE / WRITE_SIZE KiB per dispatch "
                 "and the scaled HBM bytes")
    for k in sorted(fetch):
        if not k.startswith(("void moe::", "moe::")):
            continue
        fk = float(np.median(fetch[k]))
        wk = float(np.median(write.get(k, [0.0])))
        hbm = (fk * f_scale + wk * w_scale) * 1024.0
        lines.append(f"#   {k[:100]}: {len(fetch[k])} dispatches, FETCH {fk:.0f} KiB, "
                     f"WRITE {wk:.0f} KiB, HBM {hbm / 1e6:.2f} MB")
    lines.append(f"source_hash = {source_hash('fused' if extra else 'gemm1')}")
    for key, v in rec.items():
        lines.append(f"{key} = {v:.0f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


N_CU = 256   # MI355X compute units (4 SIMDs each)
N_XCD = 8


def counter_summary(pmc_csv, out_path, workload="c4", dense=False, extra=""):
    """Per-kernel medians of every counter in one rocprofv3 --pmc CSV.
    SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs (a dense 16-bit
    product of F flops reads F / 1024: one SIMD retires 1024 bf16 flops per
    busy cycle) and GRBM_GUI_ACTIVE over the 8 XCDs, so MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024): the share of
    SIMD cycles, while the kernel ran, in which a matrix core was busy
    (padding rows of ragged tiles included).  The clock is GRBM_GUI_ACTIVE / 8
    over the dispatch's duration.  Wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES:
    the share of resident-wave cycles spent waiting on anything (memory
    counters, barriers, dependencies)."""
    import numpy as np
    rows = _counter_rows(pmc_csv)
    counters = sorted({r["Counter_Name"] for r in rows})
    per = {}
    for c in counters:
        for k, v in _per_kernel(rows, c).items():
            per.setdefault(k, {})[c] = v

    def keep(name):
        return name.startswith(("void moe::", "moe::")) or "Cijk" in name
    if dense:
        cmd = (f"python3 $R/bench.py --dense-gemm --steps 3 --warmup 1")
        what = "dense bf16 4096 x 28672 x 4096: moe_expert_ffn_down (one expert) and hipBLASLt"
    else:
        cmd = (f"python3 $R/bench.py --config {workload} --steps 3 --warmup 1 "
               f"--no-cpu-baseline {extra}").rstrip()
        what = f"workload {workload}"
    lines = [f"# rocprofv3 --pmc counters per kernel dispatch (median over dispatches), {what}",
             "# command (from /tmp, TMPDIR=/tmp, R = repository root):",
             f"#   rocprofv3 --pmc {' '.join(counters)} -f csv -d <dir> -o pmc -- {cmd}",
             f"#   python3 $R/bench.py {'--dense-gemm' if dense else '--config ' + workload} "
             f"{extra} --counter-summary <dir>/pmc_counter_collection.csv <out>".replace("  ", " "),
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs); "
             "clock = GRBM_GUI_ACTIVE / 8 / dispatch duration; "
             "wait_share = SQ_WAIT_ANY / SQ_WAVE_CYCLES"]
    dur = {}
    for r in rows:
        if r["Counter_Name"] == counters[0]:
            dur.setdefault(r["Kernel_Name"], []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for k in sorted(per, key=lambda n: n):
        if not keep(k):
            continue
        med = {c: float(np.median(v)) for c, v in per[k].items()}
        n = max(len(v) for v in per[k].values())
        parts = [f"{c} {med[c]:.4g}" for c in counters if c in med]
        d_ns = float(np.median(dur[k])) if k in dur else 0.0
        parts.append(f"duration_ns {d_ns:.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and med.get("GRBM_GUI_ACTIVE"):
            cyc = med["GRBM_GUI_ACTIVE"] / N_XCD
            parts.append(f"mfma_busy {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_CU * 4):.3f}")
            if d_ns >= 1e5:  # too coarse for short dispatches
                parts.append(f"clock_ghz {cyc / d_ns:.2f}")
        if "SQ_WAIT_ANY" in med and med.get("SQ_WAVE_CYCLES"):
            parts.append(f"wait_share {med['SQ_WAIT_ANY'] / med['SQ_WAVE_CYCLES']:.3f}")
        lines.append(f"{k[:110]}")
        lines.append(f"    dispatches {n}: " + ", ".join(parts))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def dense_gemm(args):
    """The library's GEMM and hipBLASLt on one dense bf16 product."""
    import torch
    from combine_moe_route_02_amd import _lib as L
    L.lib()
    dev = torch.device("cuda:0")
    M, N, K = 4096, 28672, 4096
    g = torch.Generator(device="cpu").manual_seed(7)
    h = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev)
    w2 = (torch.randn(1, N, K, generator=g) / K ** 0.5).to(torch.bfloat16).to(dev)
    offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    wt = w2[0]
    ours = lambda: L.moe_expert_ffn_down(offsets, N, K, 0, 1, M, w2, None, h, y)
    blas = lambda: torch.matmul(h, wt.T)

    def timed(fn):
        for _ in range(max(args.warmup if args.warmup is not None else 10, 1)):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        return t[len(t) // 2]
    t_ours, t_blas = timed(ours), timed(blas)
    ref = blas().float()
    err = ((y.float() - ref).norm() / ref.norm()).item()
    fl = 2.0 * M * N * K
    res = {"shape": [M, N, K], "dtype": "bf16", "steps": args.steps,
           "ours_ms": round(t_ours, 4), "hipblaslt_ms": round(t_blas, 4),
           "ours_frac_mfma": round(fl / t_ours / 1e9 / PEAK_MFMA_TFLOPS, 4),
           "hipblaslt_frac_mfma": round(fl / t_blas / 1e9 / PEAK_MFMA_TFLOPS, 4),
           "rel_l2_vs_hipblaslt": err}
    print(json.dumps(res), flush=True)


def stats_summary(stats_csv, out_path, workload="c2", extra=""):
    rows = _counter_rows(stats_csv)
    keys = list(rows[0].keys()) if rows else []
    name_k = "Name" if "Name" in keys else keys[0]
    lines = ["# rocprofv3 --kernel-trace --stats: per-kernel totals (ns), workload " + workload,
             "# command (from /tmp, TMPDIR=/tmp, R = repository root):",
             "#   rocprofv3 --kernel-trace --stats -f csv -d <dir> -o st -- python3 $R/bench.py "
             f"--config {workload} --no-cpu-baseline {extra}".rstrip(),
             f"#   python3 $R/bench.py --config {workload} --stats-summary "
             "<dir>/st_kernel_stats.csv <out>",
             "# input generation kernels (torch elementwise ops) run before the timed steps",
             "# " + ", ".join(["calls", "total_ns", "average_ns", "pct", "kernel"])]
    for r in rows:
        lines.append(f"{r.get('Calls', '')}, {r.get('TotalDurationNs', '')}, "
                     f"{r.get('AverageNs', '')}, {r.get('Percentage', '')}, {r[name_k][:140]}")
    # per-dispatch durations of this library's kernels from the kernel trace
    # written beside the stats: the median (the first launches of a process
    # include cold caches and page mapping)
    trace = os.path.join(os.path.dirname(stats_csv),
                         os.path.basename(stats_csv).replace("kernel_stats", "kernel_trace"))
    if trace != stats_csv and os.path.exists(trace):
        import statistics
        per = {}
        for r in _counter_rows(trace):
            if r["Kernel_Name"].startswith(("void moe::", "moe::")):
                per.setdefault(r["Kernel_Name"], []).append(
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines.append("# median ns, mean ns per dispatch (kernel trace), dispatches, kernel")
        for k, v in sorted(per.items(), key=lambda kv: -statistics.median(kv[1])):
            lines.append(f"# {statistics.median(v):.0f}, {statistics.fmean(v):.0f}, "
                         f"{len(v)}, {k[:120]}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:30]))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, inp, sample_tokens: int):
    """The oracle, as it stands, on the first S tokens of the same workload,
    timed per stage (route, dispatch, expert FFN, combine)."""
    from oracle import moe_oracle as O
    from oracle.torch_io import stored
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    # about 10-30 s of host work: the expert weights' decoding is a fixed
    # cost, so the DeepSeek-V3-like layer takes its whole batch
    S = sample_tokens or {"c1": 256, "c2": 256, "c3": 256, "c4": 16384, "c5": 128}[cfg.name]
    S = min(S, cfg.T)
    print(f"[bench] cpu oracle on {S} tokens", file=sys.stderr, flush=True)
    st = {k: (stored(v) if v is not None else None) for k, v in inp.items()}
    sub = cfg.with_(T=S)
    p = O.LayerParams(T=S, H=sub.H, E=sub.E, k=sub.k, I=sub.I, act_dtype=sub.act_dtype,
                      w_dtype=sub.w_dtype, gate=sub.gate, renorm=sub.renorm, act=sub.act,
                      e_begin=sub.e_begin, e_end=sub.e_end,
                      inv_temperature=sub.inv_temperature, min_prob=sub.min_prob,
                      fp8_dispatch=sub.fp8_dispatch)
    yr = st["y_remote"][: S * cfg.k] if st["y_remote"] is not None else None
    stages = {}
    t0 = time.perf_counter()
    O.layer_forward(p, st["x"][:S], st["w_router"], st["bias"], st["w13"], st["w2"],
                    st["w13_scale"], st["w2_scale"], yr, timings=stages)
    dt = time.perf_counter() - t0
    return {"value": round(S / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "stages_s": {k: round(v, 3) for k, v in stages.items()},
            "sample": f"first {S} of {cfg.T} tokens of the {cfg.name} layer, full "
                      f"expert weights, float64 numpy oracle on {cores} BLAS threads; "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
