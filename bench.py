#!/usr/bin/env python3
"""Benchmark of the ctconv hot path on one MI355X.

Default workload: the vocoder-style upsampler stack, bf16 storage with fp32
accumulation, N = 8: ConvTranspose1d 512->256 (k16 s8 p4) on L_in = 2000,
ELU, 256->128 (k10 s5 p3), ELU, 128->64 (k8 s4 p2).  Inputs are seeded
synthetic data with the workload's shapes and distributions; the weights are
prepacked once, outside the timed region.  One step = the three transposed
convolutions and the two ELUs, every one a libctconv kernel.

Metric: ConvTranspose TFLOP/s with F = 2*N*C_in*C_out*prod(k)*prod(L_in) per
layer, summed over the stack, divided by the wall time of the timed steps.

Prints one JSON line (rank 0).  --workload picks another workload (istft,
upsampler2d, gather2d, gather2d_dil2, upsampler1d_small) for profiling.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ConvTranspose TFLOP/s (2*N*Cin*Cout*K*Lin) and % of MFMA/HBM roofline, 1 GPU"
# ctconv_route codes of the dense layers' kernels (include/ctconv.h)
ROUTES = {"auto": 0, "gather": 2, "tiled": 3, "stream": 4}
PEAK_MFMA = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # dense TFLOP/s
PEAK_HBM = 8000.0  # GB/s
# fp32 vector arithmetic (the gather kernel's FMAs, every dtype): 256 CUs x
# 4 SIMDs x 16 lanes x 2 FMA per lane (packed) x 2 flop x 2.4 GHz
PEAK_ALU = 157.3  # TFLOP/s
FLUSH_BYTES = 512 << 20  # larger than the 256 MB MALL
ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def pcts(ms_samples):
    """p10, median and p90 of per-launch durations (ms in, us out)."""
    return [round(float(v) * 1e3, 2) for v in np.percentile(ms_samples, [10, 50, 90])]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="vocoder_stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--route", default="auto", choices=sorted(ROUTES),
                    help="kernel for the dense layers (default: the library's choice); "
                         "'gather' measures the gather fallback on the same shapes")
    ap.add_argument("--no-clock-probe", action="store_true",
                    help="skip the sustained-clock probe (about 2 ms of GPU time after the timing)")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="steps timed after a 512 MiB cache flush (at most --steps)")
    ap.add_argument("--separate-elu", action="store_true",
                    help="run the ELU between layers as its own pass instead of fusing it "
                         "into the producing layer's epilogue")
    ap.add_argument("--cpu-items", type=int, default=2,
                    help="batch items of the workload in the oracle's timed sample")
    ap.add_argument("--cpu-frames", type=int, default=0,
                    help="leading input frames per item in the sample (0: all)")
    ap.add_argument("--batch", type=int, default=0,
                    help="run the workload at this batch size instead of its own (one GPU's "
                         "share of a batch split over several GPUs)")
    ap.add_argument("--stream-frames", type=int, default=0,
                    help="also time a streaming decode (N = 1) of the 1-D stack with this many "
                         "input frames per call (12 frames = 80 ms of 24 kHz audio for the "
                         "vocoder stack) and report it under \"stream\"")
    return ap.parse_args()


def layer_geometry(wl):
    """Per layer: (layer, input spatial, output spatial, flops, algorithmic bytes)."""
    from vision_upsampler_decoders_amd import ctconv as C

    out = []
    sp = tuple(wl.in_spatial)
    es = ESIZE[wl.dtype]
    for L in wl.layers:
        osp = C.ctconv_output_shape(sp, L.kernel, L.stride, L.padding, L.output_padding,
                                    L.dilation)
        K = int(np.prod(L.kernel))
        cog = L.C_out // L.groups  # output channels per group (all of them when dense)
        flops = 2 * wl.N * L.C_in * cog * K * int(np.prod(sp))
        nbytes = es * (wl.N * L.C_in * int(np.prod(sp)) + L.C_in * cog * K
                       + (L.C_out if L.bias else 0) + wl.N * L.C_out * int(np.prod(osp)))
        out.append((L, sp, osp, flops, nbytes))
        sp = osp
    return out


def _code_only(text):
    """Source text without comments and whitespace (a comment edit is no kernel change)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return "".join("".join(out).split())


def kernel_source_digest():
    """sha256 (first 16 hex) of the HIP sources' code, comments and whitespace removed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vision_upsampler_decoders_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic measured with rocprofv3 --pmc for this kernel source, if any."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        ent = rec.get(workload)
        if ent and ent.get("kernel_digest") == kernel_source_digest():
            return ent.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, items, frames):
    """The oracle, as it stands, on the first `items` batch items of the
    workload (leading `frames` input positions when frames > 0), every layer
    and the ELUs of the stack."""
    import oracle
    from synth import inputs as I

    sp = tuple(wl.in_spatial)
    items = max(1, min(items, wl.N))
    if frames <= 0:
        sub = sp
    elif len(sp) == 1:
        sub = (min(frames, sp[0]),)
    else:  # 2-D: a band of rows
        sub = (max(1, min(sp[0], frames)), sp[1])
    x = I.gen_x(wl, N=wl.N, in_spatial=sp)[:items]
    x = x[(slice(None), slice(None)) + tuple(slice(0, v) for v in sub)]
    ws = [I.gen_w(wl, li) for li in range(len(wl.layers))]
    bs = [I.gen_bias(wl, li) for li in range(len(wl.layers))]
    flops = 0
    t0 = time.perf_counter()
    cur = x
    for li, L in enumerate(wl.layers):
        flops += (2 * items * L.C_in * (L.C_out // L.groups) * int(np.prod(L.kernel))
                  * int(np.prod(cur.shape[2:])))
        if L.groups == 1:
            cur = oracle.conv_transpose(cur, ws[li], bs[li], L.stride, L.padding,
                                        L.output_padding, L.dilation)
        else:
            cur = oracle.conv_transpose_grouped(cur, ws[li], bs[li], L.groups, L.stride,
                                                L.padding, L.output_padding, L.dilation)
        if wl.elu_between and li + 1 < len(wl.layers):
            cur = oracle.elu(cur)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"batch items 0..{items - 1} of {wl.N}, input {list(sub)} of {list(sp)}, all {len(wl.layers)} "
                      f"layer(s){' with ELU between' if wl.elu_between else ''}; "
                      f"{flops / 1e9:.2f} GFLOP in {dt:.2f} s, single-threaded float64",
            "seconds": dt, "host_nproc": os.cpu_count(), "host_cpu": cpu_model()}


def stream_latency(wl, geo, packed, biases, args, C, dcode, tdt, fuse):
    """Streaming decode at N = 1 (ctconv_stream_step per layer, each layer's
    emitted outputs feeding the next): time per call of F input frames.
    Each layer runs with padding 0 (the padded stack trims p outputs at the
    two ends of the whole stream, which does not change the work)."""
    import torch

    F = args.stream_frames
    if len(geo[0][1]) != 1 or any(g[0].kernel[0] < g[0].stride[0] for g in geo):
        return {"error": "streaming needs a 1-D stack with k >= s"}
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)
    C_in0 = geo[0][0].C_in
    x = torch.randn((1, C_in0, F), device="cuda").to(tdt)
    plan = []
    L = F
    cur = x
    for li, (Ly_, sp, osp, _, _) in enumerate(geo):
        Lr = geo[li][0]
        k, s = Lr.kernel[0], Lr.stride[0]
        Ly, Tl, ws_bytes = C.ctconv_stream_sizes(1, Lr.C_out, L, k, s, dcode)
        y = torch.empty((1, Lr.C_out, Ly), dtype=tdt, device="cuda")
        ws = torch.empty(ws_bytes // y.element_size() + 8, dtype=tdt, device="cuda")
        tails = [torch.zeros((1, Lr.C_out, max(Tl, 1)), dtype=torch.float32, device="cuda")
                 for _ in range(2)]
        act = C.ACT_ELU if (fuse and li + 1 < len(geo)) else C.ACT_NONE
        b = biases[li]
        plan.append((cur, packed[li], b, y, tails, ws, Lr.C_in, Lr.C_out, L, k, s, Tl, act))
        cur = y
        L = Ly
    fn = C.load().ctconv_stream_step

    def call(parity):
        # launches go to the current stream (the capture stream inside a graph)
        sp = int(torch.cuda.current_stream().cuda_stream)
        for (xin, pw, b, y, tails, ws, ci, co, Lc, k, s, Tl, act) in plan:
            tin, tout = tails[parity], tails[1 - parity]
            st = fn(xin.data_ptr(), pw.data_ptr(), None if b is None else b.data_ptr(),
                    y.data_ptr(), tin.data_ptr() if Tl > 0 else None,
                    tout.data_ptr() if Tl > 0 else None, ws.data_ptr(), 1, ci, co, Lc, k, s,
                    dcode, act, sp)
            assert st == 0, st

    calls = max(args.steps, 20) // 2 * 2
    for i in range(args.warmup * 2):
        call(i % 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        call(i % 2)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / calls * 1e6
    # the same two calls (the tails alternate) captured once as a HIP graph
    # and replayed: one launch of the graph instead of 12 kernel launches
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
        call(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(0)
        call(1)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls // 2):
        g.replay()
    torch.cuda.synchronize()
    us_graph = (time.perf_counter() - t0) / calls * 1e6
    out_per_call = plan[-1][3].shape[2]
    return {"N": 1, "frames_per_call": F, "outputs_per_call": int(out_per_call),
            "calls": calls, "us_per_call": round(us, 2),
            "us_per_call_graph": round(us_graph, 2), "launches_per_call": 2 * len(plan)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from synth import inputs as I
    from vision_upsampler_decoders_amd import ctconv as C

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(3)
    C.load()
    torch.cuda.set_device(0)
    wl = I.workload(args.workload)
    if args.batch > 0:
        import dataclasses
        wl = dataclasses.replace(wl, N=args.batch)
    geo = layer_geometry(wl)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]

    def dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a.astype(np.float32 if wl.dtype == "f32" else np.float16)).cuda()

    log(f"workload {wl.name}: {wl.note}")
    x = dev(I.gen_x(wl))
    packed, biases, outs, elus, weights = [], [], [], [], []
    for li, (L, sp, osp, _, _) in enumerate(geo):
        w = dev(I.gen_w(wl, li))
        # a depthwise layer reads its weight as is; a dense one its packed form
        packed.append(w if L.groups > 1 else C.prepack(w, L.stride))
        b = I.gen_bias(wl, li)
        biases.append(None if b is None else dev(b))
        outs.append(torch.empty((wl.N, L.C_out) + osp, dtype=tdt, device="cuda"))
        elus.append(torch.empty_like(outs[-1])
                    if (args.separate_elu and wl.elu_between and li + 1 < len(geo)) else None)
        weights.append(w)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)
    dcode = {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype]

    n_layers = len(geo)
    # arguments marshalled once per layer: each launch is one foreign call
    fuse = wl.elu_between and not args.separate_elu
    # dense layers go through ctconv_forward_ws: shapes with few output tiles
    # split their reduction into a workspace (deterministic); the others need none
    # (a forced kernel goes through ctconv_forward_act, without a workspace)
    forced = ROUTES[args.route]
    convs = [(C.DepthwiseConv if L.groups > 1 else C.ConvWS if forced == 0 else C.Conv)(
                 wl.N, L.C_in, L.C_out, sp, L.kernel, L.stride, L.padding, L.output_padding,
                 L.dilation, dcode, act=C.ACT_ELU if (fuse and li + 1 < len(geo)) else C.ACT_NONE,
                 **({} if (L.groups > 1 or forced == 0) else {"route": forced}))
             for li, (L, sp, osp, _, _) in enumerate(geo)]
    wspaces = [torch.empty(max(getattr(cv, "ws_bytes", 0), 16), dtype=torch.uint8, device="cuda")
               if getattr(cv, "ws_bytes", 0) > 0 else None for cv in convs]
    if any(L.groups not in (1, L.C_in) for L in wl.layers):
        raise SystemExit("grouped layers other than depthwise (groups = C_in) are not built")
    ptrs = []
    cur_ptr = x.data_ptr()
    for li in range(n_layers):
        b = biases[li]
        ptrs.append((cur_ptr, packed[li].data_ptr(), None if b is None else b.data_ptr(),
                     outs[li].data_ptr()))
        cur_ptr = outs[li].data_ptr()
        if elus[li] is not None:
            cur_ptr = elus[li].data_ptr()
    elu_fn = C.load().ctconv_elu

    def step(ev=None):
        for li in range(n_layers):
            if ev is not None:
                ev[li][0].record(stream)
            if wspaces[li] is not None:
                convs[li](*ptrs[li], sptr, wspaces[li].data_ptr(), wspaces[li].numel())
            else:
                convs[li](*ptrs[li], sptr)
            if ev is not None:
                ev[li][1].record(stream)
            if elus[li] is not None:
                if ev is not None:
                    ev[n_layers + li][0].record(stream)
                st = elu_fn(outs[li].data_ptr(), elus[li].data_ptr(), outs[li].numel(), dcode, sptr)
                if st != 0:
                    raise C.CtconvError("ctconv_elu", st)
                if ev is not None:
                    ev[n_layers + li][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: wall clock over exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch durations with HIP events on the launch stream (separate pass)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(2 * n_layers)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    layer_samples = [[evs[k][li][0].elapsed_time(evs[k][li][1]) for k in range(args.steps)]
                     for li in range(n_layers)]
    layer_ms = [float(np.mean(v)) for v in layer_samples]

    # cold regime: before each step, overwrite a 512 MiB buffer on the same stream so that
    # neither L2 nor the 256 MB MALL still holds the step's inputs or weights
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    cold_reps = max(1, min(args.steps, args.cold_reps))
    evc = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(2 * n_layers)] for _ in range(cold_reps)]
    evs_step = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                for _ in range(cold_reps)]
    for k in range(cold_reps):
        flush.fill_(float(k))
        evs_step[k][0].record(stream)
        step(evc[k])
        evs_step[k][1].record(stream)
    torch.cuda.synchronize()
    del flush
    cold_layer_samples = [[evc[k][li][0].elapsed_time(evc[k][li][1]) for k in range(cold_reps)]
                          for li in range(n_layers)]
    cold_step_ms = [evs_step[k][0].elapsed_time(evs_step[k][1]) for k in range(cold_reps)]
    elu_ms = [float(np.mean([evs[k][n_layers + li][0].elapsed_time(evs[k][n_layers + li][1])
                             for k in range(args.steps)]))
              for li in range(n_layers) if elus[li] is not None]

    # prepack (once per weight, outside the forward): event-timed per dense layer
    prepack_us = []
    for li, (L, sp, osp, _, _) in enumerate(geo):
        if L.groups > 1:
            prepack_us.append(None)
            continue
        w = weights[li]
        out_pw = torch.empty_like(packed[li])
        sz = list(L.kernel)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        C.ctconv_prepack(w.data_ptr(), out_pw.data_ptr(), len(sz), L.C_in, L.C_out, sz, L.stride,
                         dcode, sptr)
        e0.record(stream)
        for _ in range(5):
            C.ctconv_prepack(w.data_ptr(), out_pw.data_ptr(), len(sz), L.C_in, L.C_out, sz,
                             L.stride, dcode, sptr)
        e1.record(stream)
        torch.cuda.synchronize()
        assert torch.equal(out_pw, packed[li])
        prepack_us.append(round(e0.elapsed_time(e1) / 5 * 1e3, 2))
        del out_pw

    total_flops = sum(g[3] for g in geo)
    ms_per_step = wall / args.steps * 1e3
    value = total_flops / (wall / args.steps) / 1e12

    layers = []
    t_roof = 0.0
    for li, (L, sp, osp, fl, nb) in enumerate(geo):
        t = layer_ms[li] * 1e-3
        if L.groups > 1:
            route = 10 + C.ctconv_depthwise_query_kernel(
                wl.N, L.C_in, L.C_out, sp, L.kernel, L.stride, L.padding, L.output_padding,
                L.dilation, dcode)
        elif forced != 0:
            route = 2 if forced == 2 else 1
        else:
            route = C.ctconv_query_route(wl.N, L.C_in, L.C_out, sp, L.kernel, L.stride,
                                         L.padding, L.output_padding, L.dilation, dcode)
        # compute peak of the layer's kernel: MFMA for the polyphase and
        # depthwise kernels, fp32 vector ALU for the gather kernel
        alu = route == 2
        t_mfma = fl / ((PEAK_ALU if alu else PEAK_MFMA[wl.dtype]) * 1e12)
        t_hbm = nb / (PEAK_HBM * 1e9)
        t_roof += max(t_mfma, t_hbm)
        layers.append({
            "layer": li, "C_in": L.C_in, "C_out": L.C_out, "kernel": list(L.kernel),
            "stride": list(L.stride), "in": list(sp), "out": list(osp),
            "route": {1: "polyphase", 2: "gather", 11: "depthwise row-phase",
                      12: "depthwise element"}[route],
            "us": round(layer_ms[li] * 1e3, 2),
            "us_p10_p50_p90": pcts(layer_samples[li]),
            "us_cold_p10_p50_p90": pcts(cold_layer_samples[li]),
            "workspace_bytes": int(wspaces[li].numel()) if wspaces[li] is not None else 0,
            "tflops": round(fl / t / 1e12, 2), "gbps": round(nb / t / 1e9, 1),
            "bound": ("alu" if alu else "mfma") if t_mfma >= t_hbm else "hbm",
            "frac_roofline": round(max(t_mfma, t_hbm) / t, 4),
            "frac_mfma": round(t_mfma / t, 4), "frac_hbm": round(t_hbm / t, 4),
        })

    # dominant kernel: the layer launch with the most time per step
    dom = max(range(n_layers), key=lambda i: layer_ms[i])
    Ld = layers[dom]
    fl_d, nb_d = geo[dom][3], geo[dom][4]
    t_d = layer_ms[dom] * 1e-3
    if Ld["bound"] in ("mfma", "alu"):
        roof = {"bound": Ld["bound"], "achieved": round(fl_d / t_d / 1e12, 2),
                "peak": PEAK_ALU if Ld["bound"] == "alu" else PEAK_MFMA[wl.dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(nb_d / t_d / 1e9, 1), "peak": PEAK_HBM,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(f"{wl.name}/layer{dom}")
    roof["kernel"] = f"layer {dom} ({Ld['route']}), {Ld['C_in']}->{Ld['C_out']} k{Ld['kernel']} s{Ld['stride']}"
    roof["algorithmic_per_launch"] = {"flop": fl_d, "bytes": nb_d}
    roof["avg_launch_us"] = Ld["us"]
    # the same launch after a cache flush (median over the cold reps)
    t_c = float(np.median(cold_layer_samples[dom])) * 1e-3
    ach_c = fl_d / t_c / 1e12 if roof["bound"] != "hbm" else nb_d / t_c / 1e9
    roof["cold"] = {"achieved": round(ach_c, 2 if roof["bound"] != "hbm" else 1),
                    "frac": round(ach_c / roof["peak"], 4), "median_launch_us": round(t_c * 1e6, 2),
                    "reps": cold_reps}
    # The published peaks hold at 2400 MHz.  The clock the chip keeps under
    # full matrix-core load (ctconv_clock_probe, after the timed region)
    # scales the compute peaks; HBM's peak does not depend on it.
    if not args.no_clock_probe:
        mhz, probe_tf = C.sustained_clock(iters=4096)
        roof["clock"] = {"sustained_mhz": round(mhz, 1), "spec_mhz": 2400.0,
                         "probe_bf16_tflops": round(probe_tf, 1),
                         "how": "s_memtime / s_memrealtime (100 MHz) over a probe keeping every "
                                "matrix core busy"}
        if roof["bound"] != "hbm":
            roof["frac_at_sustained_clock"] = round(
                roof["achieved"] / (roof["peak"] * mhz / 2400.0), 4)


    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": wl.name, "description": wl.note, "N": wl.N,
                   "route": args.route,
                   "in_spatial": list(wl.in_spatial), "parallelism": "none (1 GPU)",
                   "elu": ("fused into the producing layer" if fuse else
                           "separate pass" if wl.elu_between else "none"),
                   "layers": [{"C_in": g[0].C_in, "C_out": g[0].C_out, "k": list(g[0].kernel),
                               "s": list(g[0].stride), "p": list(g[0].padding),
                               "op": list(g[0].output_padding), "d": list(g[0].dilation)}
                              for g in geo]},
        "roofline": roof,
        "step_roofline_fraction": round(t_roof / (ms_per_step * 1e-3), 4),
        "ms_per_step_cold_p10_p50_p90": [round(v / 1e3, 4) for v in pcts(cold_step_ms)],
        "layers": layers,
        "elu_us": [round(v * 1e3, 2) for v in elu_ms],
        "prepack_us": prepack_us,
        "gflop_per_step": round(total_flops / 1e9, 3),
    }
    if args.stream_frames > 0:
        res["stream"] = stream_latency(wl, geo, packed, biases, args, C, dcode, tdt, fuse)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_items, args.cpu_frames)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
