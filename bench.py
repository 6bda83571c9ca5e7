"""Benchmark of the MoE-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1|c2|c3|c4|c5] [--maxvio V]
                    [--combine gather|scatter] [--xperm]

The default workload is the full single-GPU layer (T=8192 H=7168 H'=2048 E=384 K=8, bf16) at
maxvio 1; the other maxvio targets (0.2, 10, 20) are timed in the same run on the same
inputs (only the routing logits change) and reported under ``skew_sweep``.

One step = one pass of the whole path over one batch of synthetic input, through the C ABI,
in the order moe_layer_forward runs it: route -> permute metadata -> gate/up + SwiGLU with
its rows gathered from x -> down -> combine (c3 passes its given routing and skips route).
``--combine scatter`` fuses the weighted combine into the down projection (fp32 atomics into
a zeroed accumulator, rounded once at the end); ``--xperm`` writes the permuted copy x_perm in
the permute and reads it in gate/up instead of gathering. Inputs and weights are resident in
HBM before the timed region starts. Each timed region is preceded by the W warmup steps and
then by untimed steps for at least ``--settle-ms`` (default 100 ms): the GPU raises its clock
over the first tens of ms of work after an idle period, and the K timed steps measure the
rate it holds under continuous work (``--settle-ms 0`` times the ramp instead).
Prints ONE JSON line. ``value`` is tokens/s of the whole layer. ``roofline`` describes the
dominant kernel (the gate/up grouped GEMM): its algorithmic flops or bytes per launch over
its average duration measured with HIP events on the launch stream during the timed steps.
``cpu_baseline`` is the float64 oracle timed on the host on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + grouped-FFN TFLOP/s as % of MFMA peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3      # fp32 vector
PEAK_HBM_GBS = 8000.0         # HBM3E

DESCR = {
    "c1": "tiny fp32 MoE layer T=64 H=128 H'=64 E=8 K=2, logits = x.Wr",
    "c2": "bf16 MoE layer T=4096 H=2048 H'=1024 E=64 K=6, uniform routing",
    "c3": "bf16 expert-parallel rank share: 65536 rows (T=8192 K=8) over 52 expert slots "
          "(1260/1261 rows each), H=7168 H'=2048, routing given",
    "c4": "bf16 MoE layer T=8192 H=7168 H'=2048 E=384 K=8, skewed routing",
    "c5": "fp8 x MXFP4 MoE layer T=8192 H=7168 H'=2048 E=384 K=8, maxvio 1",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed repetitions for at least this long before each timed region")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one at a time after evicting the caches (0: skip)")
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--maxvio", type=float, default=1.0, help="skew target for c4 (the headline)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="c4: skip timing the other maxvio targets (0.2, 1, 10, 20) beside the headline")
    ap.add_argument("--cpu-sample-experts", type=int, default=0,
                    help="experts in the oracle timing sample (0: whole layer when it is small)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--combine", default="gather", choices=["gather", "scatter"],
                    help="deterministic gather-reduce (default) or the scatter-add fused into down")
    ap.add_argument("--shared-hs", type=int, default=0,
                    help="also time moe_layer_forward and moe_layer_forward_shared (a shared "
                         "expert of this intermediate size on the same or a side stream); "
                         "reported under 'layer_with_shared_expert', the headline value stays "
                         "the routed layer")
    ap.add_argument("--pad", type=int, default=1,
                    help="static-capacity layout: pad every expert group to a multiple of this many rows")
    ap.add_argument("--bf16-input", action="store_true",
                    help="c5 only: bf16 activations quantised to fp8 1x128 inside the timed step")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of the step captured as a HIP graph")
    ap.add_argument("--backward", action="store_true",
                    help="also time moe_layer_backward (bf16 layers), reported under 'backward'")
    ap.add_argument("--ffn", default="auto", choices=["auto", "two", "fused"],
                    help="bf16: gate/up and down as two persistent launches or as one "
                         "(moe_grouped_ffn_fused, or moe_grouped_ffn_fused_scatter with --combine "
                         "scatter, reported as stage 'ffn'); auto picks as moe_layer_forward does: "
                         "one launch when T*K <= 256*E and the combine is the gather")
    ap.add_argument("--mxfp4-layout", default="paired", choices=["plain", "paired"],
                    help="MXFP4 weights (c5): repacked once before timing into the paired layout "
                         "(moe_pack_mxfp4_pairs, MOE_MXFP4_PAIRED; the default, about 1 %% faster "
                         "at c5) or read in their stored layout")
    ap.add_argument("--xperm", action="store_true",
                    help="materialise x_perm in the permute instead of gathering rows in gate/up")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known bytes) a few times, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(steps):
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": steps + 1, "copy_ms": ms, "copy_gbs": 2 * n / ms / 1e6}), flush=True)


def source_hash(*names):
    """Hash of the kernel sources' code: comments and whitespace are dropped first, so that
    only a change to the code itself invalidates the stored traffic counters."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixture_experts_layer_counting_amd", "csrc", n)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def settle(fn, ms, torch):
    """Untimed repetitions of fn for at least `ms` of wall time. After an idle period the GPU
    raises its clock over the first tens of ms of work (c2: 0.45 ms per step in the first 25
    steps, a steady 0.375 ms from about 30 ms on); the timed steps that follow then run at the
    rate the GPU holds under continuous work."""
    if ms <= 0:
        return 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def load_traffic(kernel, workload, khash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the kernel as it is now (same source hash); otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
        ent = table[f"{kernel}@{workload}"]
        if ent.get("source_hash") != khash:
            return None
        return float(ent["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs the MoE layer on exactly one GPU; expert parallelism "
              "over several GPUs is designed but not implemented (see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return

    import torch

    import mixture_experts_layer_counting_amd as moe
    from workloads import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()   # fail loudly if the HIP library is missing
    quant = args.bf16_input and args.config == "c5"
    w = gen.config(args.config, device=dev, maxvio=args.maxvio if args.config == "c4" else None,
                   shared_hs=args.shared_hs, act="bf16" if quant else None)
    T, H, Hp, E, K = w.T, w.H, w.Hp, w.E, w.K
    M = T * K
    pad = max(args.pad, 1)
    MR = moe.moe_padded_capacity(T, E, K, pad)   # rows of the permuted buffers (M when pad = 1)
    x_in, x_in_sf = w.x, w.x_sf
    if quant:   # the layer's own activation format from here on: fp8 with 1x128 scales
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xq_sf = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
        w.act, w.x, w.x_sf = "fp8", xq, xq_sf
    DT = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3, "mxfp4": moe.MOE_MXFP4}
    TD = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    hf = "fp8" if w.act == "fp8" else w.act
    # The weights as the step reads them. With --mxfp4-layout paired the MXFP4 codes are
    # repacked once, before any timing (like loading the weights), into the layout of
    # MOE_MXFP4_PAIRED; the oracle keeps reading the stored layout of w.
    wg_g, wu_g, wd_g, wgt_g = w.w_gate, w.w_up, w.w_down, DT[w.wgt]
    if w.wgt == "mxfp4" and args.mxfp4_layout == "paired":
        def pack(t, n_cols, k_red):
            o = torch.empty_like(t)
            moe.moe_pack_mxfp4_pairs(t, o, E, n_cols, k_red, None)
            return o
        wg_g, wu_g, wd_g = pack(w.w_gate, Hp, H), pack(w.w_up, Hp, H), pack(w.w_down, H, Hp)
        wgt_g = moe.MOE_MXFP4_PAIRED
        torch.cuda.synchronize()
    yf = "f32" if w.act == "f32" else "bf16"
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    topk_idx = torch.empty((T, K), **i32) if w.logits is not None else w.topk_idx
    topk_w = torch.empty((T, K), **f32) if w.logits is not None else w.topk_w
    counts = torch.empty(E, **i32)
    cu = torch.empty(E + 1, **i32)
    pos = torch.empty((T, K), **i32)
    row_src = torch.empty(MR, **i32)
    scatter = args.combine == "scatter"
    x_perm = torch.empty((MR, H), dtype=TD[w.act], device=dev) if args.xperm else None
    # fp8: the permutation writes the block-major scales also when the rows are gathered
    x_perm_sf = torch.empty((H // 128, MR), **f32) if w.act == "fp8" else None
    row_w = torch.empty(MR, **f32) if scatter else None
    h = torch.empty((MR, Hp), dtype=TD[hf], device=dev)
    h_sf = torch.empty((Hp // 128, MR), **f32) if w.act == "fp8" else None
    y = torch.empty((MR, H), dtype=TD[yf], device=dev) if not scatter else None
    out = torch.empty((T, H), dtype=TD[w.out], device=dev)
    acc = (out if w.out == "f32" else torch.empty((T, H), **f32)) if scatter else None
    nws = moe.moe_permute_workspace_bytes(T, E, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    if args.ffn == "auto":
        args.ffn = "fused" if (w.act == "bf16" and not scatter and not args.xperm and pad == 1
                               and M <= 256 * E and H % 256 == 0 and Hp % 128 == 0
                               and min(H, Hp) >= 256) else "two"
    fused = args.ffn == "fused"
    if fused:
        if w.act != "bf16" or args.xperm or pad != 1:
            sys.exit("bench.py: --ffn fused takes the bf16 layer with gathered rows and no padding")
        nws_f = moe.moe_grouped_ffn_fused_workspace_bytes(M, E, Hp)
        ws_f = torch.empty(nws_f, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # combine: acc zero + store (scatter); ffn: gate/up and down as one launch (--ffn fused)
    stages = ["quantize", "route", "permute", "gate_up", "down", "ffn", "combine"]
    ev = {s: [] for s in stages}
    stage_fns = {}

    def step(record):
        def mark(name, fn):
            stage_fns[name] = fn
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                ev[name].append((a, b))
            else:
                fn()
        if quant:
            mark("quantize", lambda: moe.moe_quantize_fp8(x_in, moe.MOE_BF16, T, H, xq, xq_sf, None))
        if w.logits is not None:   # routing and permutation in one call (stage "permute")
            mark("permute", lambda: moe.moe_route_permute(w.logits, w.x, w.x_sf, DT[w.act], T, H, E, K, pad,
                                                          topk_idx, topk_w, counts, cu, pos, row_src, row_w,
                                                          x_perm, x_perm_sf, ws, nws, None))
        else:
            mark("permute", lambda: moe.moe_permute_padded(w.x, w.x_sf, DT[w.act], topk_idx, topk_w, T, H, E,
                                                           K, pad, counts, cu, pos, row_src, row_w, x_perm,
                                                           x_perm_sf, ws, nws, None))
        if fused and scatter:
            # the weighted combine in the single launch's down epilogue, into the fp32 accumulator
            mark("combine", lambda: acc.zero_())
            mark("ffn", lambda: moe.moe_grouped_ffn_fused_scatter(w.x, DT[w.act], row_src, T, K, cu, M, E, H,
                                                                  Hp, wg_g, wu_g, wd_g, wgt_g,
                                                                  row_w, acc, ws_f, nws_f, None))
            if acc is not out:
                mark("combine", lambda: out.copy_(acc))
            return
        if fused:
            mark("ffn", lambda: moe.moe_grouped_ffn_fused(w.x, DT[w.act], row_src, T, K, cu, M, E, H, Hp,
                                                          wg_g, wu_g, wd_g, wgt_g, y, DT[yf],
                                                          ws_f, nws_f, None))
            mark("combine", lambda: moe.moe_combine(y, DT[yf], pos, topk_w, T, H, K, out, DT[w.out], None))
            return
        if args.xperm:
            mark("gate_up", lambda: moe.moe_ffn_gate_up(x_perm, x_perm_sf, DT[w.act], cu, MR, E, H, Hp,
                                                        wg_g, wu_g, w.sf_gate, w.sf_up,
                                                        wgt_g, h, h_sf, None))
        else:
            mark("gate_up", lambda: moe.moe_ffn_gate_up_gather(w.x, None, x_perm_sf, DT[w.act], row_src, T,
                                                               K, cu, MR, E, H, Hp, wg_g, wu_g,
                                                               w.sf_gate, w.sf_up, wgt_g, h, h_sf, None))
        if not scatter:
            mark("down", lambda: moe.moe_ffn_down(h, h_sf, DT[hf], cu, MR, E, H, Hp, wd_g, w.sf_down,
                                                  wgt_g, y, DT[yf], None))
            mark("combine", lambda: moe.moe_combine(y, DT[yf], pos, topk_w, T, H, K, out, DT[w.out], None))
        else:
            mark("combine", lambda: acc.zero_())
            mark("down", lambda: moe.moe_ffn_down_scatter(h, h_sf, DT[hf], cu, MR, E, H, Hp, wd_g,
                                                          w.sf_down, wgt_g, row_src, row_w, T, K,
                                                          acc, None))
            if acc is not out:
                mark("combine", lambda: out.copy_(acc))

    for _ in range(args.warmup):
        step(False)
    settle(lambda: step(False), args.settle_ms, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step_eager = elapsed * 1e3 / args.steps
    eager_out = out.clone()
    # Headline timing: the same step captured once as a HIP graph and replayed, so the host
    # launch gaps between its kernels are gone (every kernel of the step still runs each
    # replay). The per-stage times above come from the eager pass.
    graph_check = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(False)
        for _ in range(args.warmup):
            graph.replay()
        settle(graph.replay, args.settle_ms, torch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        graph_check = bool(torch.equal(out, eager_out)) if not scatter else \
            float((out.float() - eager_out.float()).abs().max() / eager_out.float().abs().max().clamp_min(1e-30))
    ms_step = elapsed * 1e3 / args.steps
    # Cold-cache step time, reported beside the headline: each step replayed alone right after
    # a 1 GiB read, which evicts the 256 MB memory-side cache (MALL) and the L2s, so nothing the
    # previous step touched is served from them. Median over the steps; one replay per event
    # pair, so the graph's launch is inside each sample.
    cold_ms = None
    if not args.no_graph and args.cold_steps > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        samples = []
        for _ in range(args.cold_steps):
            flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            graph.replay()
            b.record()
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b))
        cold_ms = float(statistics.median(samples))
        del flush
    # Cold-cache stage times of the HBM-bound stages: the permute (routing included when it
    # comes from logits) and the combine, each run alone right after the same cache eviction,
    # median over --cold-steps. The step has run before, so every input of the stage is in place.
    stage_ms_cold = {}
    if args.cold_steps > 0 and not scatter:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        for name in ("permute", "combine"):
            samples = []
            for _ in range(args.cold_steps):
                flush.sum()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                stage_fns[name]()
                b.record(stream)
                torch.cuda.synchronize()
                samples.append(a.elapsed_time(b))
            stage_ms_cold[name] = float(statistics.median(samples))
        del flush
    # per stage: total event time of the stage in a step (the scatter combine has two parts),
    # median over the timed steps
    def per_step(name):
        if not ev[name]:
            return 0.0
        per = len(ev[name]) // args.steps
        tot = [sum(a.elapsed_time(b) for a, b in ev[name][i * per:(i + 1) * per]) for i in range(args.steps)]
        return float(statistics.median(tot))
    stage_ms = {s: per_step(s) for s in stages}

    # ---------------------------------------------------------------- algorithmic units
    cnt = counts.cpu().numpy()
    active = int((cnt > 0).sum())
    ab = {"f32": 4, "bf16": 2, "fp8": 1}[w.act]
    hb = {"f32": 4, "bf16": 2, "fp8": 1}[hf]
    yb = 4 if yf == "f32" else 2
    ob = 4 if w.out == "f32" else 2
    if w.wgt == "mxfp4":
        wmat = H * Hp // 2 + H * Hp // 32          # packed e2m1 + e8m0 scales
    else:
        wmat = H * Hp * {"f32": 4, "bf16": 2}[w.wgt]
    xsf_b = M * (H // 128) * 4 if w.act == "fp8" else 0
    hsf_b = M * (Hp // 128) * 4 if w.act == "fp8" else 0
    gu_flops = 4.0 * M * H * Hp
    dn_flops = 2.0 * M * H * Hp
    gu_bytes = M * H * ab + xsf_b + 2 * active * wmat + M * Hp * hb + hsf_b
    dn_bytes = M * Hp * hb + hsf_b + active * wmat + M * H * yb
    # permute: topk_idx read; pos, row_src (and row_w from topk_w) written; + the row copy;
    # with routing in the same call, the logits read and topk_idx / topk_w written instead
    perm_bytes = M * 4 + 2 * M * 4 + (2 * M * 4 if scatter else 0)
    if w.logits is not None:
        perm_bytes += T * E * 4 + M * 4
    if w.act == "fp8":   # x_sf read, the block-major permuted scales written
        perm_bytes += T * (H // 128) * 4 + xsf_b
    if args.xperm:
        perm_bytes += T * H * ab + M * H * ab
    if scatter:   # zero the fp32 accumulator, then round it once into out (bf16)
        comb_bytes = T * H * 4 + ((T * H * 4 + T * H * ob) if w.out != "f32" else 0)
        dn_bytes = M * Hp * hb + hsf_b + active * wmat + M * 4 * 2   # + the fp32 adds, M*H*4
    else:
        comb_bytes = M * H * yb + T * H * ob
    peak_flops = {"f32": PEAK_FP32_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS}[w.act]
    # the dominant kernel: gate/up, or with --ffn fused the single launch that runs gate/up and down
    if fused:
        k_ms, k_flops, k_bytes = stage_ms["ffn"], gu_flops + dn_flops, gu_bytes + dn_bytes
        kname = "ffn_fused (gate/up + SwiGLU and down in one persistent launch)"
        kfiles, tkernel = ("ffn_fused.hip",), "ffn_fused_scatter" if scatter else "ffn_fused"
    else:
        k_ms, k_flops, k_bytes = stage_ms["gate_up"], gu_flops, gu_bytes
        kname = "ffn_gate_up (grouped GEMM gate+up, SwiGLU epilogue)"
        kfiles = ({"bf16": "ffn_bf16.hip", "fp8": "ffn_fp8.hip", "f32": "ffn_f32.hip"}[w.act],)
        tkernel = "gate_up" if args.xperm else "gate_up_gather"
    k_s = k_ms / 1e3
    t_mfma = k_flops / (peak_flops * 1e12)
    t_hbm = k_bytes / (PEAK_HBM_GBS * 1e9)
    khash = source_hash(*kfiles, "tile_sched.h", "moe_common.h", "lds_dma.h")
    wl_key = f"{args.config}_maxvio{args.maxvio:g}" if args.config == "c4" else args.config
    traffic = load_traffic(tkernel, wl_key, khash)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": k_flops / k_s / 1e12, "peak": peak_flops, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": k_bytes / k_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = kname
    roof["per_launch"] = {"flops": k_flops, "bytes": k_bytes, "avg_ms": k_ms,
                          "mfma_time_at_peak_ms": t_mfma * 1e3, "hbm_time_at_peak_ms": t_hbm * 1e3}
    # the other roofline beside the binding one: the kernel's rate against the MFMA peak of its
    # input type (the metric's "% of MFMA peak") and against the HBM peak
    roof["mfma_frac"] = k_flops / k_s / 1e12 / peak_flops
    roof["hbm_frac"] = k_bytes / k_s / 1e9 / PEAK_HBM_GBS

    ffn_ms = stage_ms["ffn"] if fused else stage_ms["gate_up"] + stage_ms["down"]
    ffn_tflops = (gu_flops + dn_flops) / (ffn_ms / 1e3) / 1e12
    rates = {"ffn_tflops": ffn_tflops} if fused else {
        "gate_up_tflops": gu_flops / (stage_ms["gate_up"] / 1e3) / 1e12,
        "down_tflops": dn_flops / (stage_ms["down"] / 1e3) / 1e12}
    line = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms_step,
        "ms_per_step_eager": ms_step_eager,
        "ms_per_step_cold_cache": cold_ms,
        "timing": "HIP graph replay of the whole step" if not args.no_graph else "eager launches",
        "graph_replay_matches_eager": graph_check,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8xmxfp4"}[w.act],
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {"workload": f"{args.config}: {DESCR[args.config]}", "T": T, "H": H, "Hp": Hp,
                   "E": E, "K": K, "act": w.act, "wgt": w.wgt, "combine": args.combine,
                   "x_perm": "materialised" if args.xperm else "gathered in gate/up",
                   "ffn": "one persistent launch" if fused else "two persistent launches",
                   "pad": pad, "input": "bf16, quantised in the step" if quant else w.act,
                   "mxfp4_layout": args.mxfp4_layout if w.wgt == "mxfp4" else None},
        "rows": {"real": int(cnt.sum()), "in_groups": int(cu[-1].item()), "buffer": int(MR)},
        "grouped_ffn_tflops": ffn_tflops,
        "grouped_ffn_frac_of_mfma_peak": ffn_tflops / peak_flops,
        "stage_ms": stage_ms,
        "stage_rates": {
            **rates,
            "permute_gbs": perm_bytes / (stage_ms["permute"] / 1e3) / 1e9,
            "combine_gbs": comb_bytes / (stage_ms["combine"] / 1e3) / 1e9,
        },
        "stage_ms_cold": stage_ms_cold,
        "stage_rates_cold": {f"{k}_gbs": {"permute": perm_bytes, "combine": comb_bytes}[k] / (v / 1e3) / 1e9
                             for k, v in stage_ms_cold.items()},
        "routing": {"maxvio": float(cnt.max() / (T * K / E) - 1.0), "active_experts": active,
                    "rows_min": int(cnt.min()), "rows_max": int(cnt.max()),
                    "maxvio_target": w.meta.get("maxvio_target"),
                    # per-expert real rows and the rows of its group as laid out (padded when
                    # --pad > 1): both, so padding never hides in the rates
                    "counts": [int(v) for v in cnt],
                    "group_rows": [int(v) for v in (cu[1:] - cu[:-1]).cpu().tolist()]},
        "roofline": roof,
    }
    if fused:
        # control words of the last single-launch call (layout in include/moe.h)
        o = (M * Hp * 2 + 255) // 256 * 256
        c = ws_f[o:o + 64].view(torch.int32).cpu().tolist()
        line["ffn_fused_ctl"] = {"error": c[8], "tiles": c[9], "not_prefetched": c[10],
                                 "from_other_queues": c[11]}
    if args.shared_hs:
        line["layer_with_shared_expert"] = time_fused(w, args, moe, torch)
    if args.backward and w.act == "bf16" and w.wgt == "bf16":
        line["backward"] = time_backward(w, args, moe, torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args, out, y if pad == 1 else None)
    if args.config == "c4" and not args.no_sweep:
        line["skew_sweep"] = skew_sweep(w, args, step, graph if not args.no_graph else None, ev, counts,
                                        stage_ms, ms_step, torch, out, y if pad == 1 else None)
    print(json.dumps(line), flush=True)


def sweep_stages(args):
    return ("permute", "ffn", "combine") if args.ffn == "fused" else ("permute", "gate_up", "down", "combine")


def skew_sweep(w, args, step, graph, ev, counts, stage_ms, ms_step, torch, out=None, y=None):
    """The same layer at every maxvio target: only the routing logits change (copied into the
    buffer the step and its graph read), x and the weights stay. Per target: the step time
    (graph replays, as the headline), tokens/s and the per-stage times (eager pass, HIP events
    on the launch stream), and unless --no-cpu-baseline the oracle timed on a shorter sample
    (about 2.5 s of host work) with its comparison against the GPU's rows. The headline target
    reuses the headline's figures (its oracle timing is the line's cpu_baseline)."""
    from workloads import gen
    base = w.logits.clone()
    head_cnt = counts.cpu().numpy()          # the headline routing, before any target replaces it
    res = {}
    for mv in gen.SKEW_TARGETS:
        if mv == args.maxvio:
            cnt = head_cnt
            res[f"{mv:g}"] = {"ms_per_step": ms_step, "tokens_per_s": w.T / (ms_step / 1e3),
                              "stage_ms": {k: stage_ms[k] for k in sweep_stages(args)},
                              "maxvio": float(cnt.max() / (w.T * w.K / w.E) - 1.0),
                              "rows_min": int(cnt.min()), "rows_max": int(cnt.max())}
            continue
        w.logits.copy_(gen.with_maxvio(w, mv).logits)
        for _ in range(args.warmup):
            step(False)
        settle(lambda: step(False), args.settle_ms, torch)
        for k in ev:
            ev[k].clear()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        st = {}
        for name in sweep_stages(args):
            per = len(ev[name]) // args.steps
            st[name] = float(statistics.median(
                [sum(a.elapsed_time(b) for a, b in ev[name][i * per:(i + 1) * per]) for i in range(args.steps)]))
        run = graph.replay if graph is not None else (lambda: step(False))
        for _ in range(args.warmup):
            run()
        settle(run, args.settle_ms, torch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        cnt = counts.cpu().numpy()
        res[f"{mv:g}"] = {"ms_per_step": ms, "tokens_per_s": w.T / (ms / 1e3), "stage_ms": st,
                          "maxvio": float(cnt.max() / (w.T * w.K / w.E) - 1.0),
                          "rows_min": int(cnt.min()), "rows_max": int(cnt.max())}
        if not args.no_cpu_baseline and out is not None:
            res[f"{mv:g}"]["cpu_baseline"] = cpu_baseline(w, args, out, y, budget_s=2.5)
    w.logits.copy_(base)
    ms = [v["ms_per_step"] for v in res.values()]
    res["slowest_over_fastest"] = max(ms) / min(ms)
    return res


def time_fused(w, args, moe, torch):
    """Whole-layer entry points timed end to end (events on the launch stream): the routed
    layer alone, and with a shared expert of size Hs on a side stream (overlapped) or on the
    same stream (serial)."""
    DT = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3, "mxfp4": moe.MOE_MXFP4}
    comb = moe.MOE_COMBINE_SCATTER_ATOMIC if args.combine == "scatter" else moe.MOE_COMBINE_GATHER
    d = moe.LayerDesc(w.T, w.H, w.Hp, w.E, w.K, DT[w.act], DT[w.wgt], DT[w.out], comb)
    n = max(moe.moe_layer_shared_workspace_bytes(d, w.Hs), moe.moe_layer_workspace_bytes(d))
    ws = torch.empty(n, dtype=torch.uint8, device=w.x.device)
    out = torch.empty((w.T, w.H), dtype={"f32": torch.float32, "bf16": torch.bfloat16}[w.out],
                      device=w.x.device)
    side = torch.cuda.Stream()
    stream = torch.cuda.current_stream()

    def routed():
        moe.moe_layer_forward(d, w.x, w.x_sf, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up,
                              w.w_down, w.sf_gate, w.sf_up, w.sf_down, out, ws, n)

    def shared(side_stream):
        moe.moe_layer_forward_shared(d, w.Hs, w.x, w.x_sf, w.x_shared, w.logits, w.topk_idx, w.topk_w,
                                     w.w_gate, w.w_up, w.w_down, w.sf_gate, w.sf_up, w.sf_down,
                                     w.ws_gate, w.ws_up, w.ws_down, out, ws, n, side_stream=side_stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        settle(fn, args.settle_ms, torch)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_routed = timed(routed)
    ms_serial = timed(lambda: shared(None))
    ms_side = timed(lambda: shared(side))
    return {"Hs": w.Hs, "ms_layer_forward": ms_routed, "ms_layer_forward_shared_serial": ms_serial,
            "ms_layer_forward_shared_side_stream": ms_side,
            "shared_expert_ms_hidden": ms_serial - ms_side,
            "tokens_per_s_with_shared": w.T / (ms_side / 1e3)}


def time_backward(w, args, moe, torch):
    """moe_layer_backward end to end (forward recomputed inside), HIP events around graph
    replays. Work: the recomputed forward (6 M H H') + down dgrad (2 M H H') + gate/up
    dgrad (4 M H H') + the three weight gradients (6 M H H') = 18 M H H' flops."""
    dev = w.x.device
    d = moe.LayerDesc(w.T, w.H, w.Hp, w.E, w.K, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16, 0)
    n = moe.moe_layer_backward_workspace_bytes(d)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    g = torch.Generator(device="cpu").manual_seed(8)
    dout = torch.randn((w.T, w.H), generator=g).to(torch.bfloat16).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dx = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    dwg = torch.empty((w.E, w.H, w.Hp), **f32)
    dwu = torch.empty((w.E, w.H, w.Hp), **f32)
    dwd = torch.empty((w.E, w.Hp, w.H), **f32)
    dtw = torch.empty((w.T, w.K), **f32)
    dl = torch.empty((w.T, w.E), **f32) if w.logits is not None else None

    def run():
        moe.moe_layer_backward(d, w.x, w.logits, w.topk_idx, w.topk_w, w.w_gate, w.w_up, w.w_down, dout, dx,
                               dwg, dwu, dwd, dtw, dl, ws, n)
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    graph.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = 18.0 * w.T * w.K * w.H * w.Hp
    return {"ms": ms, "tokens_per_s": w.T / (ms / 1e3), "tflops": flops / (ms / 1e3) / 1e12,
            "frac_of_mfma_peak": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "work": "forward recomputed + dgrad + wgrad (18 M H H' flops), bf16, HIP graph replay"}


def cpu_baseline(w, args, gpu_out, gpu_y=None, budget_s=10.0):
    """The oracle, as it stands, on the host: whole layer when small, else routing + permute +
    combine for all tokens and the FFN for a sample of experts, scaled to all experts. The
    GPU's result is compared with the oracle's: the whole output when every expert is in the
    sample, else the permuted rows y of the sampled experts."""
    import numpy as np
    import torch

    from oracle import moe_oracle as O
    from workloads import to_numpy_bits

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    xb = to_numpy_bits(w.x)
    x = O.decode_activations(xb, w.act, to_numpy_bits(w.x_sf))
    fp8 = w.act == "fp8"

    def wfn(e):
        if w.wgt == "mxfp4":
            return (O.decode_mxfp4(to_numpy_bits(w.w_gate[e]), to_numpy_bits(w.sf_gate[e])),
                    O.decode_mxfp4(to_numpy_bits(w.w_up[e]), to_numpy_bits(w.sf_up[e])),
                    O.decode_mxfp4(to_numpy_bits(w.w_down[e]), to_numpy_bits(w.sf_down[e])))
        dec = (lambda a: np.asarray(a, np.float64)) if w.wgt == "f32" else O.decode_bf16
        return dec(to_numpy_bits(w.w_gate[e])), dec(to_numpy_bits(w.w_up[e])), dec(to_numpy_bits(w.w_down[e]))

    n_sample = args.cpu_sample_experts or (w.E if w.T * w.H <= 4096 * 2048 else 8)
    n_sample = min(n_sample, w.E)
    experts = None
    sampled_rows, y_sampled = [], []

    def one_pass():
        """One oracle pass over the sample; returns (seconds it stands for, measured seconds, out)."""
        nonlocal experts
        t0 = time.perf_counter()
        if w.logits is not None:
            idx, wts = O.route_topk(to_numpy_bits(w.logits), w.K)
        else:
            idx, wts = to_numpy_bits(w.topk_idx), to_numpy_bits(w.topk_w).astype(np.float64)
        counts, cu = O.count_offsets(idx, w.E)
        pos, row_src = O.permute(idx, w.E)
        tok = row_src // w.K
        t1 = time.perf_counter()
        experts = list(range(w.E)) if n_sample == w.E else \
            [int(e) for e in np.linspace(0, w.E - 1, n_sample).round().astype(int)]
        y_rows = np.zeros((w.T * w.K, w.H))
        t_ffn = 0.0
        for e in experts:
            lo, hi = int(cu[e]), int(cu[e + 1])
            if hi == lo:
                continue
            s = time.perf_counter()
            wg, wu, wd = wfn(e)
            _, y_rows[lo:hi] = O.expert_ffn(x[tok[lo:hi]], wg, wu, wd, fp8)
            t_ffn += time.perf_counter() - s
        t2 = time.perf_counter()
        out = O.combine(y_rows, pos, wts)
        t3 = time.perf_counter()
        scale = w.E / len(experts)
        sampled_rows.clear()
        sampled_rows.extend((int(cu[e]), int(cu[e + 1])) for e in experts)
        y_sampled.clear()
        y_sampled.extend(y_rows[lo:hi] for lo, hi in sampled_rows)
        return (t1 - t0) + t_ffn * scale + (t3 - t2), (t1 - t0) + t_ffn + (t3 - t2), out

    # repeat the pass until about budget_s of host work has been measured (at most 20 passes)
    totals, measured, ref = [], 0.0, None
    while not totals or (measured < budget_s and len(totals) < 20):
        tot, meas, ref = one_pass()
        totals.append(tot)
        measured += meas
    total = sum(totals) / len(totals)
    scale = w.E / len(experts)
    res = {"value": w.T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "host_cpus": os.cpu_count(), "measured_s": measured, "passes": len(totals),
           "sample": (f"whole layer ({w.T} tokens, all {w.E} experts), mean of {len(totals)} passes"
                      if n_sample == w.E else
                      f"routing + permute + combine for all {w.T} tokens; expert FFN for "
                      f"{len(experts)} of {w.E} experts (all their rows), FFN time scaled by "
                      f"{scale:.1f}; mean of {len(totals)} passes")}
    if n_sample == w.E:
        got = gpu_out.detach().cpu()
        got = got.double().numpy() if got.dtype == torch.float32 else got.to(torch.float64).numpy()
        res["gpu_vs_oracle_rel_err"] = float(np.abs(got - ref).max() / np.abs(ref).max())
        res["gpu_vs_oracle_what"] = "out, every token"
    elif gpu_y is not None:
        errs, n = [], 0
        for (lo, hi), yr in zip(sampled_rows, y_sampled):
            if hi == lo:
                continue
            got = gpu_y[lo:hi].detach().cpu()
            got = got.double().numpy() if got.dtype == torch.float32 else got.to(torch.float64).numpy()
            errs.append(float(np.abs(got - yr).max() / np.abs(yr).max()))
            n += hi - lo
        res["gpu_vs_oracle_rel_err"] = max(errs) if errs else None
        res["gpu_vs_oracle_what"] = (f"y_rows of the {len(errs)} sampled experts ({n} rows), "
                                     "max over experts of max|err| / max|ref|")
    return res


if __name__ == "__main__":
    main()
