"""Benchmark of the quantized MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload nvfp4_zipf] [--tokens T]
                    [--no-cpu-baseline] [--no-regimes] [--no-stack]

A step is one full forward of the expert layer (routing, grouping, fused
dequant gate/up GEMM + SwiGLU, down GEMM, combine) over one batch of synthetic
tokens with every input already resident in HBM.  Consecutive steps cycle
through several distinct layers' weights (>= 1.5 GiB in total, more than the
256 MB last-level cache), so every step streams its expert weights from HBM as
a real model's consecutive layers would.

The headline line is the largest batch: NVFP4 weights, 16384 tokens with
Zipf-skewed routing (the prefill regime, bound by the matrix units).  Beside it:

* ``regimes``: the decode layer (INT4, 1 / 8 / 64 tokens, bound by HBM), the
  FP8 prefill layer (4096 tokens), and the same FP8 layer with dynamic 1x128
  FP8 activations on the FP8 matrix units (W8A8), the NVFP4 layer with 4-bit
  activations (W4A4, 16384 tokens), each with the median, p10 and p90 of
  per-step times with the weights cycled through the sets, with one set
  repeated (warm caches) and after a 1 GiB flush (cold caches), plus the
  decode batches replayed from a captured HIP graph;
* ``with_router``: the decode (64 tokens) and FP8 prefill layers driven from the
  BF16 gate's weight, router GEMM and top-k fused in one kernel, against the
  router-logits kernel followed by the logits-driven forward;
* ``import``: checkpoint import of one layer per format (FineGrainedFP8,
  auto_gptq INT4, compressed-tensors NVFP4 source layouts), against HBM;
* ``stack48``: the 48-layer stack (24 FP8 + 24 INT4 layers chained with
  residual adds) at 64 and 2048 tokens, eager and graph-captured;
* ``cpu_baseline``: the float64 oracle on a bounded sample of the headline
  batch, on the host's cores.

``roofline`` rates the dominant kernel of each line, timed live with HIP events
that the runtime takes at the kernel's own start and end on the stream it runs
on (``hipExtLaunchKernel``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense FP16/BF16 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
STAGES = ("route", "permute", "gate_up", "down", "combine")
EVERY = 4  # bracket the dominant kernel with events in one step of every EVERY
CSRC = os.path.join(ROOT, "weight_quantized_moe_amd", "csrc")
METRIC = "MoE layer tokens/s + % roofline (HBM GB/s decode, MFMA util prefill)"


def packed_bytes(fmt, n, k):
    if fmt == "int4_g128":
        return n * k // 2 + n * (k // 128) * 2
    if fmt == "fp8_b128":
        return n * k + (n // 128) * (k // 128) * 4
    return n * k // 2 + n * (k // 16) + 4


def source_hash(files=None) -> str:
    """Hash of the kernel sources (all of csrc/, or the named files in it and
    the headers they include)."""
    names = sorted(os.listdir(CSRC)) if files is None else sorted(set(files) | {"device.h", "internal.h"})
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel's source changed since it was taken
    (the summary names the source file and its hash)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    f = re.search(r"source_file\s*=\s*([\w.]+)", text)
    m = re.search(r"source_hash\s*=\s*(\w+)", text)
    b = re.search(r"hbm_bytes_per_launch\s*=\s*([0-9.eE+]+)", text)
    if not f or not m or not b or m.group(1) != source_hash([f.group(1)]):
        return None
    return float(b.group(1))


def kernel_work(fmt, E, H, I, k, T, touched):
    """Algorithmic bytes and flops.  Bytes: the packed weights + scales of the
    touched experts, the hidden rows read once (gate/up) and the output written
    once (down); the intermediate h and the per-slot partials are the
    implementation's own traffic and are not counted.  Flops: 6 H I per routed
    row (4 H I gate/up, 2 H I down); no padding rows, no unpack, no SwiGLU."""
    R = T * k
    w13_b, w2_b = packed_bytes(fmt, 2 * I, H), packed_bytes(fmt, H, I)
    return {
        "bytes": {"gate_up": touched * w13_b + T * H * 2, "down": touched * w2_b + T * H * 2},
        "flops": {"gate_up": 4 * H * I * R, "down": 2 * H * I * R},
        "path_bytes": touched * (w13_b + w2_b) + 2 * T * H * 2 + T * E * 4,
        "path_flops": 6 * H * I * R,
    }


def pct(vals, q):
    s = sorted(vals)
    return s[min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))]


def new_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:          # torch creates the HIP event on first record
        e.record()
    return evs


class LayerBench:
    """One workload's layer: several weight sets (cycled so they stream from
    HBM), its synthetic batch, workspace and output."""

    def __init__(self, wl, T, dev, min_bytes=1.5 * 2 ** 30, seed0=1000, share=None, w8a8=False,
                 w4a4=False):
        import numpy as np
        import torch
        from weight_quantized_moe_amd import Layer, synth
        self.wl, self.T, self.dev, self.w8a8, self.w4a4 = wl, T, dev, w8a8, w4a4
        E, H, I, k, fmt = wl.experts, wl.hidden, wl.inter, wl.top_k, wl.fmt
        layer_bytes = E * (packed_bytes(fmt, 2 * I, H) + packed_bytes(fmt, H, I))
        self.n_sets = max(2, math.ceil(min_bytes / layer_bytes))
        self.layers, self.first_np = [], None
        if share is not None:            # the same weight sets at another batch size
            self.n_sets, self.layers, self.first_np = share.n_sets, share.layers, share.first_np
        for li in range(len(self.layers), self.n_sets):
            t13 = synth.random_packed_torch(fmt, E, 2 * I, H, seed0 + 2 * li, dev)
            t2 = synth.random_packed_torch(fmt, E, H, I, seed0 + 1 + 2 * li, dev)
            if li == 0:
                self.first_np = tuple(None if a is None else a.cpu().numpy() for a in (*t13, *t2))
            self.layers.append(Layer(fmt, t13[0], t13[1], t2[0], t2[1], k,
                                     w13_gscale=t13[2], w2_gscale=t2[2]))
        self.logits_np = synth.router_logits(wl.wid, 0, T, E, wl.logits)
        self.x_np = synth.hidden_bf16(wl.wid, 0, T, H)
        self.logits = torch.from_numpy(self.logits_np).to(dev)
        self.x = torch.from_numpy(self.x_np.view(np.int16)).to(dev).view(torch.bfloat16)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.ws = self.layers[0].workspace(T, dev)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.layers[0].forward(self.logits, self.x, out=self.out, workspace=self.ws,
                               probe={"expert_offsets": offs})
        torch.cuda.synchronize()
        self.touched = int((torch.diff(offs) > 0).sum().item())
        self.work = kernel_work(fmt, E, H, I, k, T, self.touched)
        if w4a4:
            # calibrated activation global scales (448 * 6 over the largest
            # value): the hidden rows, and the intermediate of a 16-bit pass
            h = torch.empty((T * k, I), dtype=torch.float16, device=dev)
            self.layers[0].forward(self.logits, self.x, out=self.out, workspace=self.ws, probe={"h": h})
            self.gx = 448 * 6 / float(self.x.float().abs().max())
            self.gh = 448 * 6 / float(h.float().abs().max())
            del h

    def fwd(self, i, events=None):
        lay = self.layers[i % self.n_sets]
        if self.w4a4:
            lay.forward_w4a4(self.logits, self.x, self.gx, self.gh, out=self.out, workspace=self.ws,
                             events=events)
            return
        f = lay.forward_w8a8 if self.w8a8 else lay.forward
        f(self.logits, self.x, out=self.out, workspace=self.ws, events=events)

    def stages(self, n):
        """Average per-stage time (ms) over n steps (its own run: ten event
        records per step)."""
        import torch
        bev = [new_events(2 * len(STAGES)) for _ in range(n)]
        for i in range(n):
            self.fwd(i, bev[i])
        torch.cuda.synchronize()
        return {s: sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in bev) / n
                for j, s in enumerate(STAGES)}

    def timed(self, steps, warmup, dom):
        """Exactly `steps` steps between two events (sets cycled); the dominant
        kernel bracketed by runtime-taken kernel events in every EVERY-th step."""
        import torch
        for i in range(warmup):
            self.fwd(i)
        jd = STAGES.index(dom)
        sampled = list(range(0, steps, EVERY))
        dev_ev = {i: new_events(2) for i in sampled}
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            ev = None
            if i in dev_ev:
                ev = [None] * (2 * len(STAGES))
                ev[2 * jd], ev[2 * jd + 1] = dev_ev[i]
            self.fwd(i, ev)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = [a.elapsed_time(b) for a, b in dev_ev.values()]
        return dict(ms=start.elapsed_time(end) / steps, wall_ms=wall * 1e3 / steps,
                    dom_ms=sum(kern) / len(kern), dom_med_ms=pct(kern, 0.5))

    def per_step(self, iters, mode, flush=None):
        """Per-step times (us), each step between its own event pair: `cycled`
        (weight sets in turn), `warm` (set 0 every time) or `cold` (set 0 after
        an untimed write of a 1 GiB buffer, which evicts L2 and the MALL)."""
        import torch
        evs = [new_events(2) for _ in range(iters)]
        torch.cuda.synchronize()
        for i in range(iters):
            if mode == "cold":
                flush.fill_(i & 0xFF)
            evs[i][0].record()
            self.fwd(i if mode == "cycled" else 0)
            evs[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    def graph_us(self, reps):
        """Per-step time (us) of the steps replayed from one captured HIP graph
        that holds one forward per weight set, in turn."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(self.n_sets):
                self.fwd(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(self.n_sets):
                self.fwd(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = new_events(2)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * self.n_sets)


def roofline(lb, dom, dom_ms, decode):
    wl = lb.wl
    secs = dom_ms * 1e-3
    if decode:
        algo = lb.work["bytes"][dom]
        achieved = algo / secs / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        algo = lb.work["flops"][dom]
        achieved = algo / secs / 1e12
        peak = PEAK_FP8_TFLOPS if lb.w8a8 else PEAK_FP16_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        if lb.w8a8:
            roof["mfma_dtype"] = "fp8 (e4m3 x e4m3)"
            roof["frac_of_fp16_peak"] = round(achieved / PEAK_FP16_TFLOPS, 4)
    tag = f"{dom}_{wl.fmt}{'_w8a8' if lb.w8a8 else ''}{'_w4a4' if lb.w4a4 else ''}_T{lb.T}"
    roof["traffic"] = counter_traffic(tag)
    roof["kernel"] = dom
    roof["kernel_us"] = round(dom_ms * 1e3, 2)
    roof["algorithmic_bytes" if decode else "algorithmic_flops"] = algo
    return roof


def is_decode(wl, T):
    return T * wl.top_k <= 16 * wl.experts


def regime_line(lb, iters, flush, graph):
    """Distribution of per-step times for one workload and batch size."""
    stage_ms = lb.stages(min(iters, 30))
    dom = max(("gate_up", "down"), key=lambda s: stage_ms[s])
    t = lb.timed(iters, 5, dom)
    out = {"workload": lb.wl.name + ("_w8a8" if lb.w8a8 else "") + ("_w4a4" if lb.w4a4 else ""),
           "format": lb.wl.fmt, "tokens": lb.T,
           "touched_experts": lb.touched,
           "tokens_per_s": round(lb.T / (t["ms"] * 1e-3), 1), "us_per_step": round(t["ms"] * 1e3, 2)}
    for mode in ("cycled", "warm", "cold"):
        v = lb.per_step(iters, mode, flush)
        out[f"{mode}_us"] = {"median": round(pct(v, 0.5), 2), "p10": round(pct(v, 0.1), 2),
                             "p90": round(pct(v, 0.9), 2)}
    if graph:
        out["graph_us_per_step"] = round(lb.graph_us(max(10, iters // lb.n_sets)), 2)
    out["stage_us"] = {s: round(v * 1e3, 2) for s, v in stage_ms.items()}
    out["roofline"] = roofline(lb, dom, t["dom_ms"], is_decode(lb.wl, lb.T))
    return out


def router_line(lb, iters):
    """The layer driven from the BF16 gate's weight: moe_quant_forward_with_router
    (router GEMM and top-k in one kernel) against the two-kernel pipeline
    moe_quant_router_logits + moe_quant_forward, same layer, batch and weight
    sets.  The fused routing kernel is rated against HBM: the hidden rows read
    once, the gate read once, the top-k ids and weights written (prefill also
    writes the FP16 rows it stages for the GEMM)."""
    import torch
    from weight_quantized_moe_amd import router_logits, synth
    wl, T, dev = lb.wl, lb.T, lb.dev
    gen = torch.Generator(device=dev).manual_seed(11)
    gate = (torch.randn(wl.experts, wl.hidden, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    lg = torch.empty((T, wl.experts), dtype=torch.float32, device=dev)

    def fused(i, events=None):
        lb.layers[i % lb.n_sets].forward_with_router(gate, lb.x, out=lb.out, workspace=lb.ws,
                                                     events=events)

    def unfused(i):
        router_logits(lb.x, gate, out=lg)
        lb.layers[i % lb.n_sets].forward(lg, lb.x, out=lb.out, workspace=lb.ws)

    res = {"workload": wl.name, "tokens": T}
    for name, fn in (("fused_us_per_step", fused), ("logits_kernel_then_forward_us_per_step", unfused)):
        for i in range(5):
            fn(i)
        e0, e1 = new_events(2)
        torch.cuda.synchronize()
        e0.record()
        for i in range(iters):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / iters, 2)
    n = min(iters, 30)
    bev = [new_events(2 * len(STAGES)) for _ in range(n)]
    for i in range(n):
        fused(i, bev[i])
    torch.cuda.synchronize()
    route_us = sum(e[0].elapsed_time(e[1]) for e in bev) / n * 1e3
    nbytes = T * wl.hidden * 2 + wl.experts * wl.hidden * 2 + T * wl.top_k * 8
    if not is_decode(wl, T):
        nbytes += T * wl.hidden * 2 + T * 4
    res["fused_route_stage_us"] = round(route_us, 2)
    res["fused_route_roofline"] = {"bound": "hbm", "algorithmic_bytes": nbytes,
                                   "achieved": round(nbytes / route_us / 1e3, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(nbytes / route_us / 1e3 / PEAK_HBM_GBS, 4)}
    return res


def import_bench(dev, reps=3):
    """Checkpoint import of a whole layer at the Clef shape (128 experts,
    moe_quant_import_expert per expert) from synthetic source tensors of each
    format's checkpoint layout, rated against HBM: the source bytes read plus
    the packed bytes written."""
    import torch
    from weight_quantized_moe_amd import import_expert
    E, H, I = 128, 2048, 768
    out = []
    g = torch.Generator(device=dev).manual_seed(13)
    u8 = lambda *s: torch.randint(0, 256, s, dtype=torch.uint8, device=dev, generator=g)  # noqa: E731
    for fmt in ("fp8_b128", "int4_g128", "nvfp4_g16"):
        kd = 1 if fmt == "fp8_b128" else 2
        if fmt == "int4_g128":
            dst = (u8(E, 2 * I, H // 2), torch.zeros(E, 2 * I, H // 128, dtype=torch.float16, device=dev),
                   u8(E, H, I // 2), torch.zeros(E, H, I // 128, dtype=torch.float16, device=dev), None, None)

            def src(n, k):
                qw = u8(k // 8, n, 4).view(torch.int32).view(k // 8, n)
                qz = torch.full((k // 128, n // 8), 0x77777777, dtype=torch.int32, device=dev)
                return qw, qz, torch.rand(k // 128, n, device=dev, generator=g).to(torch.float16)
        elif fmt == "fp8_b128":
            dst = (u8(E, 2 * I, H), torch.zeros(E, 2 * I // 128, H // 128, device=dev), u8(E, H, I),
                   torch.zeros(E, H // 128, I // 128, device=dev), None, None)

            def src(n, k):
                return u8(n, k), torch.rand(n // 128, k // 128, device=dev, generator=g)
        else:
            dst = (u8(E, 2 * I, H // 2), u8(E, 2 * I, H // 16), u8(E, H, I // 2), u8(E, H, I // 16),
                   torch.ones(E, device=dev), torch.ones(E, device=dev))

            def src(n, k):
                return u8(n, k // 2), u8(n, k // 16), 2.5
        srcs = [(src(I, H), src(I, H), src(H, I)) for _ in range(8)]   # 8 distinct source experts
        nbytes = 2 * E * (packed_bytes(fmt, 2 * I, H) + packed_bytes(fmt, H, I))   # read + write
        if fmt == "int4_g128":   # the zero points are read as well
            nbytes += E * 4 * ((H // 128) * (2 * I) // 8 + (I // 128) * H // 8)
        times = []
        for r in range(reps + 1):
            e0, e1 = new_events(2)
            torch.cuda.synchronize()
            e0.record()
            for e in range(E):
                sg, su, sd = srcs[e % 8]
                import_expert(fmt, dst, e, sg, su, sd)
            e1.record()
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1) * 1e3)
        us = pct(times, 0.5)
        out.append({"format": fmt, "experts": E, "us_per_layer": round(us, 1), "bytes": nbytes,
                    "GB_s": round(nbytes / us / 1e3, 1), "frac_of_8TB_s": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                    "launches_per_expert": 9 if fmt == "int4_g128" else (7 if fmt == "nvfp4_g16" else 6)})
        del dst, srcs
    return out


def stack_bench(dev, reps):
    """All 48 layers back to back (layers 0-23 FP8, 24-47 INT4, residual adds),
    eager and replayed from one captured HIP graph, at 64 and 2048 tokens."""
    import numpy as np
    import torch
    from weight_quantized_moe_amd import Layer, synth
    wl = synth.WORKLOADS["stack48"]
    E, H, I, k, L = wl.experts, wl.hidden, wl.inter, wl.top_k, wl.layers
    layers = []
    for li in range(L):
        fmt = synth.stack_layer_format(li)
        t13 = synth.random_packed_torch(fmt, E, 2 * I, H, 5000 + 2 * li, dev)
        t2 = synth.random_packed_torch(fmt, E, H, I, 5001 + 2 * li, dev)
        layers.append((fmt, Layer(fmt, t13[0], t13[1], t2[0], t2[1], k)))
    res = {"layers": L, "formats": "0-23 fp8_b128, 24-47 int4_g128"}
    for T in wl.tokens:
        lgs = [torch.from_numpy(synth.router_logits(wl.wid, li, T, E)).to(dev) for li in range(L)]
        x0 = torch.from_numpy(synth.hidden_bf16(wl.wid, 0, T, H).view(np.int16)).to(dev).view(torch.bfloat16)
        ws = max((lay.workspace(T, dev) for _, lay in layers[:1] + layers[-1:]), key=lambda w: w.numel())
        bufs = [x0.clone(), torch.empty_like(x0)]
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        touched, roof_s, hbm_bytes, flops = [], 0.0, 0, 0
        for li, (fmt, lay) in enumerate(layers):
            lay.forward(lgs[li], x0, out=bufs[1], workspace=ws, probe={"expert_offsets": offs})
            torch.cuda.synchronize()
            n = int((torch.diff(offs) > 0).sum().item())
            touched.append(n)
            w = kernel_work(fmt, E, H, I, k, T, n)
            hbm_bytes += w["path_bytes"]
            flops += w["path_flops"]
            roof_s += max(w["path_bytes"] / (PEAK_HBM_GBS * 1e9), w["path_flops"] / (PEAK_FP16_TFLOPS * 1e12))

        def chain():
            for li, (_, lay) in enumerate(layers):
                src, dst = bufs[li & 1], bufs[(li + 1) & 1]
                lay.forward(lgs[li], src, residual=src, out=dst, workspace=ws)

        # one checked pass: which layers saturate an FP16 intermediate, and the
        # size of the residual stream at the end
        bufs[0].copy_(x0)
        saturated = []
        for li, (_, lay) in enumerate(layers):
            src, dst = bufs[li & 1], bufs[(li + 1) & 1]
            lay.forward(lgs[li], src, residual=src, out=dst, workspace=ws)
            if lay.check(ws):
                saturated.append(li)
        final_rms = bufs[L & 1].float().square().mean().sqrt().item()
        bufs[0].copy_(x0)
        chain()
        torch.cuda.synchronize()
        evs = [new_events(2) for _ in range(reps)]
        for r in range(reps):
            evs[r][0].record()
            chain()
            evs[r][1].record()
        torch.cuda.synchronize()
        eager = [a.elapsed_time(b) for a, b in evs]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain()
        g.replay()
        torch.cuda.synchronize()
        evs = [new_events(2) for _ in range(reps)]
        for r in range(reps):
            evs[r][0].record()
            g.replay()
            evs[r][1].record()
        torch.cuda.synchronize()
        graph = [a.elapsed_time(b) for a, b in evs]
        med_e, med_g = pct(eager, 0.5), pct(graph, 0.5)
        res[f"T{T}"] = {
            "tokens": T, "touched_experts_mean": round(sum(touched) / L, 1),
            "eager_ms": {"median": round(med_e, 4), "p10": round(pct(eager, 0.1), 4),
                         "p90": round(pct(eager, 0.9), 4)},
            "graph_ms": {"median": round(med_g, 4), "p10": round(pct(graph, 0.1), 4),
                         "p90": round(pct(graph, 0.9), 4)},
            "per_layer_us": {"eager": round(med_e * 1e3 / L, 2), "graph": round(med_g * 1e3 / L, 2)},
            "tokens_per_s_graph": round(T / (med_g * 1e-3), 1),
            "algorithmic_bytes": hbm_bytes, "algorithmic_flops": flops,
            "roofline_ms": round(roof_s * 1e3, 4),
            "frac_of_roofline_graph": round(roof_s * 1e3 / med_g, 4),
            "hbm_GBps_graph": round(hbm_bytes / (med_g * 1e-3) / 1e9, 1),
            "saturated_layers": saturated, "final_residual_rms": round(final_rms, 4),
        }
        del g
    return res


def cpu_baseline(lb, budget_s=10.0, max_tokens=4096):
    """The oracle as it stands on a contiguous sample of the headline batch
    (its first tokens, same layer and routing), repeated until ~budget_s."""
    import numpy as np
    from oracle import formats, moe
    wl = lb.wl
    E, H, I, k, fmt = wl.experts, wl.hidden, wl.inter, wl.top_k, wl.fmt
    w, s, g, w_, s_, g_ = lb.first_np
    lay = moe.Layer(formats.Packed(fmt, w, s, g, 2 * I, H), formats.Packed(fmt, w_, s_, g_, H, I), k)
    info = {}
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info = {"blas": f"{blas[0].get('internal_api')} {blas[0].get('version')}",
                    "threads": blas[0].get("num_threads")}
    except Exception:  # pragma: no cover
        pass
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    sample = np.arange(min(lb.T, max_tokens))
    done, t0 = 0, time.perf_counter()
    while True:
        moe.moe_forward(lay, lb.logits_np, lb.x_np, tokens=sample)
        done += len(sample)
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    # the GEMM-only part of the same sample: both projections over the
    # already dequantized weights of the experts it routes to
    ids, _ = moe.route(lb.logits_np[sample], k)
    perm = moe.permute(ids, E)
    x = moe.bf16_bits_to_f64(lb.x_np[sample])
    deq = {e: (formats.dequantize_expert(lay.w13, e), formats.dequantize_expert(lay.w2, e))
           for e in range(E) if perm.offsets[e + 1] > perm.offsets[e]}
    t1 = time.perf_counter()
    for e, (d13, d2) in deq.items():
        rows = x[perm.sorted_token_ids[perm.offsets[e]:perm.offsets[e + 1]]]
        gu = rows @ d13.T
        (gu[:, :I] * gu[:, I:]) @ d2.T
    gemm_s = time.perf_counter() - t1
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": info.get("threads", 1),
            "kind": "oracle", "cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)),
            "blas": info.get("blas", "unknown"),
            "gemm_only_tokens_per_s": round(len(sample) / gemm_s, 1),
            "sample": f"{done} tokens: the first {len(sample)} tokens of the {lb.T}-token batch "
                      f"({fmt}, {wl.logits} logits), float64 NumPy per-expert loop incl. "
                      f"dequantization, routing and combine, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="nvfp4_zipf")
    ap.add_argument("--tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-regimes", action="store_true", help="skip the decode / FP8 prefill lines")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer stack")
    ap.add_argument("--iters", type=int, default=100, help="per-step samples of each regime line")
    ap.add_argument("--router", action="store_true",
                    help="only time the router logits kernel (moe_quant_router_logits) at H 2048, E 128")
    ap.add_argument("--vendor-bmm", action="store_true",
                    help="only time torch.bmm (hipBLASLt) FP16 at the prefill expert-GEMM shapes, for reference")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer is data parallel over tokens; DESIGN.md describes how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_quantized_moe_amd import load_library, synth

    dev = torch.device("cuda:0")
    if args.router:
        load_library()
        print(json.dumps({"kernel": "router logits (moe_quant_router_logits), BF16 MFMA, FP32 out",
                          "results": router_bench(dev, max(args.steps, 20))}))
        return
    if args.vendor_bmm:
        print(json.dumps({"reference": "torch.bmm FP16 (hipBLASLt), not this library",
                          "results": vendor_bmm(dev, max(args.steps, 20))}))
        return
    load_library()
    wl = synth.WORKLOADS[args.workload]
    if wl.fmt == "stack":
        raise SystemExit("the 48-layer stack is timed in the 'stack48' part of the default run")
    T = args.tokens or max(wl.tokens)
    lb = LayerBench(wl, T, dev)
    decode = is_decode(wl, T)
    stage_ms = lb.stages(min(args.steps, 20))
    dom = max(("gate_up", "down"), key=lambda s: stage_ms[s])
    r = lb.timed(args.steps, args.warmup, dom)
    print(f"# headline {wl.name} T={T}: {r['ms'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    res = {
        "metric": METRIC,
        "value": round(T / (r["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc, bf16 io",
        "data": "synthetic (seeded packed codes, N(0,1) activations and logits)",
        "config": {"workload": wl.name, "format": wl.fmt, "tokens": T, "hidden": wl.hidden,
                   "intermediate": wl.inter, "experts": wl.experts, "top_k": wl.top_k,
                   "logits": wl.logits, "touched_experts": lb.touched, "weight_sets_cycled": lb.n_sets},
        "roofline": roofline(lb, dom, r["dom_ms"], decode),
        "path_roofline": {"bytes": lb.work["path_bytes"], "flops": lb.work["path_flops"],
                          "hbm_GBps": round(lb.work["path_bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                          "tflops": round(lb.work["path_flops"] / (r["ms"] * 1e-3) / 1e12, 2),
                          "frac_of_mfma_peak": round(lb.work["path_flops"] / (r["ms"] * 1e-3) / 1e12
                                                     / PEAK_FP16_TFLOPS, 4)},
        "stage_us": {s: round(v * 1e3, 2) for s, v in stage_ms.items()},
        "wall_ms_per_step": round(r["wall_ms"], 4),
    }
    flush = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    if not args.no_regimes:
        res["regimes"] = []
        prev = None
        for name, T2 in (("decode_int4", 1), ("decode_int4", 8), ("decode_int4", 64),
                         ("prefill_fp8", 4096)):
            share = prev if prev is not None and prev.wl.name == name else None
            other = LayerBench(synth.WORKLOADS[name], T2, dev, share=share)
            line = regime_line(other, args.iters, flush, graph=is_decode(other.wl, T2))
            res["regimes"].append(line)
            print(f"# {name} T={T2}: {line['us_per_step']} us/step", file=sys.stderr, flush=True)
            if T2 in (64, 4096):
                res.setdefault("with_router", []).append(router_line(other, args.iters))
            prev = other
        # W8A8 block FP8: the FP8 prefill layer with dynamic FP8 activations
        w8 = LayerBench(synth.WORKLOADS["prefill_fp8"], 4096, dev, share=prev, w8a8=True)
        line = regime_line(w8, args.iters, flush, graph=False)
        res["regimes"].append(line)
        print(f"# prefill_fp8 W8A8 T=4096: {line['us_per_step']} us/step", file=sys.stderr, flush=True)
        del prev, other, w8
        # NVFP4 W4A4: the NVFP4 layer with 4-bit activations (calibrated global scales)
        nv = synth.WORKLOADS["nvfp4_zipf"]
        same = lb.wl.name == nv.name and lb.T == 16384
        w4 = LayerBench(nv, 16384, dev, share=lb if same else None, w4a4=True)
        line = regime_line(w4, args.iters, flush, graph=False)
        res["regimes"].append(line)
        print(f"# nvfp4_zipf W4A4 T=16384: {line['us_per_step']} us/step", file=sys.stderr, flush=True)
        del w4
    res["import"] = import_bench(dev)
    print("# import done", file=sys.stderr, flush=True)
    if not args.no_stack:
        res["stack48"] = stack_bench(dev, max(5, args.steps // 2))
        print("# stack48 done", file=sys.stderr, flush=True)
    del flush
    # plain copy of known size: reference reading for HBM byte counters
    src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(lb)
    print(json.dumps(res))


def vendor_bmm(dev, steps):
    """Reference point, not part of the layer: the vendor dense FP16 batched GEMM
    (torch.bmm, hipBLASLt) at the expert-GEMM shapes of the prefill workloads,
    with uniform rows per expert and weights already in FP16."""
    import torch
    out = []
    for name, (E, M, N, K) in (("gate/up, 256 rows per expert", (128, 256, 1536, 2048)),
                               ("down, 256 rows per expert", (128, 256, 2048, 768)),
                               ("gate/up, 1024 rows per expert", (128, 1024, 1536, 2048)),
                               ("gate/up, one GEMM of 32768 rows", (1, 32768, 1536, 2048))):
        a = torch.randn(E, M, K, device=dev, dtype=torch.float16).contiguous()
        b = torch.randn(E, K, N, device=dev, dtype=torch.float16).contiguous()
        for _ in range(5):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.bmm(a, b)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        tf = 2.0 * E * M * N * K / us / 1e6
        out.append({"gemm": name, "shape_EMNK": [E, M, N, K], "us": round(us, 2),
                    "TFLOP_s": round(tf, 1), "frac_of_2.5PF": round(tf / 2500.0, 4)})
    return out


def router_bench(dev, steps):
    """The router logits kernel alone (moe_quant_router_logits) at the layer's
    shape, H 2048 and E 128, for the decode and prefill batch sizes.  It is
    bound by HBM: x [T, H] and the gate [E, H] in BF16, logits [T, E] in FP32,
    2 T H E FLOP on the BF16 matrix units."""
    import torch
    from weight_quantized_moe_amd import router_logits
    H, E = 2048, 128
    out = []
    gen = torch.Generator(device=dev).manual_seed(7)
    w = (torch.randn(E, H, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    for T in (64, 4096, 16384):
        x = torch.randn(T, H, device=dev, generator=gen).to(torch.bfloat16)
        lg = torch.empty(T, E, device=dev, dtype=torch.float32)
        for _ in range(5):
            router_logits(x, w, out=lg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            router_logits(x, w, out=lg)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = T * H * 2 + E * H * 2 + T * E * 4
        gbs = nbytes / us / 1e3
        out.append({"tokens": T, "us": round(us, 2), "bytes": nbytes, "GB_s": round(gbs, 1),
                    "frac_of_8TB_s": round(gbs / 8000.0, 4),
                    "TFLOP_s": round(2.0 * T * H * E / us / 1e6, 1)})
    return out


if __name__ == "__main__":
    main()
