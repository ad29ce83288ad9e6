"""Benchmark of the quantized MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_int4] [--tokens T]

A step is one full forward of the expert layer (routing, grouping, fused
dequant gate/up GEMM + SwiGLU, down GEMM, combine) over one batch of synthetic
tokens with every input already resident in HBM.  Consecutive steps cycle
through several distinct layers' weights (>= 1.5 GiB in total, more than the
256 MB last-level cache), so every step streams its expert weights from HBM as
a real model's consecutive layers would.

Prints one JSON line: whole-step tokens/s, the roofline position of the
dominant kernel (timed live with HIP events on the stream it runs on, which
the library has the runtime take at the kernel's own start and end), and the
CPU oracle timed on a bounded sample of the same workload.
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
STAGES = ("route", "permute", "gate_up", "down", "combine")
EVERY = 8  # bracket the dominant kernel with events in one step of every EVERY
KERNEL_SRC = os.path.join(ROOT, "weight_quantized_moe_amd", "csrc", "gemm.hip")


def packed_bytes(fmt, n, k):
    if fmt == "int4_g128":
        return n * k // 2 + n * (k // 128) * 2
    if fmt == "fp8_b128":
        return n * k + (n // 128) * (k // 128) * 4
    return n * k // 2 + n * (k // 16) + 4


def source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.dirname(KERNEL_SRC))):
        with open(os.path.join(os.path.dirname(KERNEL_SRC), name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash\s*=\s*(\w+)", text)
    b = re.search(r"hbm_bytes_per_launch\s*=\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != source_hash():
        return None
    return float(b.group(1))


def cpu_baseline(layer_np, logits, x, budget_s=12.0):
    """The oracle as it stands, on whole batches of the same workload, repeated
    until ~budget_s of CPU work."""
    import numpy as np
    from oracle import moe
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    T = x.shape[0]
    sample = np.arange(min(T, 64))
    done, t0 = 0, time.perf_counter()
    while True:
        moe.moe_forward(layer_np, logits, x, tokens=sample)
        done += len(sample)
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} tokens ({len(sample)}-token batches of the same layer, "
                      f"float64 NumPy per-expert loop incl. dequantization), {el:.1f} s"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_int4")
    ap.add_argument("--tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also time every batch size of the workload")
    ap.add_argument("--router", action="store_true",
                    help="only time the router logits kernel (moe_quant_router_logits) at H 2048, E 128")
    ap.add_argument("--vendor-bmm", action="store_true",
                    help="only time torch.bmm (hipBLASLt) FP16 at the prefill expert-GEMM shapes, for reference")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer is data parallel over tokens; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from weight_quantized_moe_amd import Layer, load_library, synth

    if args.router:
        load_library()
        print(json.dumps({"kernel": "router logits (moe_quant_router_logits), BF16 MFMA, FP32 out",
                          "results": router_bench(torch.device("cuda:0"), max(args.steps, 20))}))
        return
    if args.vendor_bmm:
        print(json.dumps({"reference": "torch.bmm FP16 (hipBLASLt), not this library",
                          "results": vendor_bmm(torch.device("cuda:0"), max(args.steps, 20))}))
        return
    load_library()
    wl = synth.WORKLOADS[args.workload]
    if wl.fmt == "stack":
        raise SystemExit("use --workload decode_int4 | prefill_fp8 | nvfp4_zipf")
    E, H, I, k, fmt = wl.experts, wl.hidden, wl.inter, wl.top_k, wl.fmt
    T = args.tokens or max(wl.tokens)
    dev = torch.device("cuda:0")

    w13_b = packed_bytes(fmt, 2 * I, H)
    w2_b = packed_bytes(fmt, H, I)
    layer_bytes = E * (w13_b + w2_b)
    n_layers = max(2, math.ceil(1.5 * 2 ** 30 / layer_bytes))
    layers, np_layers = [], []
    for li in range(n_layers):
        t13, ts13, tg13 = synth.random_packed_torch(fmt, E, 2 * I, H, 1000 + 2 * li, dev)
        t2, ts2, tg2 = synth.random_packed_torch(fmt, E, H, I, 1001 + 2 * li, dev)
        if li == 0 and not args.no_cpu_baseline:
            to_np = lambda a: None if a is None else a.cpu().numpy()  # noqa: E731
            np_layers = tuple(map(to_np, (t13, ts13, tg13, t2, ts2, tg2)))
        layers.append(Layer(fmt, t13, ts13, t2, ts2, k, w13_gscale=tg13, w2_gscale=tg2))

    def run_config(T, steps, warmup):
        logits_np = synth.router_logits(wl.wid, 0, T, E, wl.logits)
        x_np = synth.hidden_bf16(wl.wid, 0, T, H)
        logits = torch.from_numpy(logits_np).to(dev)
        x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws = layers[0].workspace(T, dev)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        layers[0].forward(logits, x, out=out, workspace=ws, probe={"expert_offsets": offs})
        torch.cuda.synchronize()
        touched = int((torch.diff(offs) > 0).sum().item())
        for i in range(warmup):
            layers[i % n_layers].forward(logits, x, out=out, workspace=ws)

        def new_events(n):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            for e in evs:          # torch creates the HIP event on first record
                e.record()
            return evs

        # stage breakdown (its own run: ten event records per step)
        nb = min(steps, 50)
        bev = [new_events(2 * len(STAGES)) for _ in range(nb)]
        for i in range(nb):
            layers[i % n_layers].forward(logits, x, out=out, workspace=ws, events=bev[i])
        torch.cuda.synchronize()
        stage_ms = {s: sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in bev) / nb
                    for j, s in enumerate(STAGES)}
        dom = max(("gate_up", "down"), key=lambda s: stage_ms[s])
        jd = STAGES.index(dom)
        # timed region: K steps.  HIP events on the layer's stream bracket the
        # dominant kernel in every EVERY-th step (an event pair costs a few
        # microseconds of GPU time, so bracketing every launch would inflate
        # the step time it is part of).
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
            layers[i % n_layers].forward(logits, x, out=out, workspace=ws, events=ev)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(end) / steps
        dom_ms = sum(a.elapsed_time(b) for a, b in dev_ev.values()) / len(dev_ev)
        return dict(T=T, ms=ms, wall_ms=wall * 1e3 / steps, stage_ms=stage_ms, touched=touched,
                    dom=dom, dom_ms=dom_ms, logits=logits_np, x=x_np)

    r = run_config(T, args.steps, args.warmup)
    R = T * k
    touched = r["touched"]
    # algorithmic work (SURVEY/DESIGN definitions)
    path_bytes = touched * (w13_b + w2_b) + T * H * 2 * 2 + T * E * 4
    flops = 6 * H * I * R
    kern_bytes = {
        "gate_up": touched * w13_b + T * H * 2 + R * I * 2,
        "down": touched * w2_b + R * I * 2 + R * H * 4,
    }
    kern_flops = {"gate_up": 4 * H * I * R, "down": 2 * H * I * R}
    dom = r["dom"]
    dom_s = r["dom_ms"] * 1e-3
    decode = R <= 16 * E
    if decode:
        achieved = kern_bytes[dom] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = kern_flops[dom] / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4)}
    tag = f"{dom}_{fmt}_T{T}"
    traffic = counter_traffic(tag)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["kernel_us"] = round(r["dom_ms"] * 1e3, 2)
    roof["algorithmic_bytes" if decode else "algorithmic_flops"] = \
        kern_bytes[dom] if decode else kern_flops[dom]

    res = {
        "metric": "MoE layer tokens/s + % roofline (HBM GB/s decode, MFMA util prefill)",
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
        "config": {"workload": wl.name, "format": fmt, "tokens": T, "hidden": H,
                   "intermediate": I, "experts": E, "top_k": k, "logits": wl.logits,
                   "touched_experts": touched, "weight_sets_cycled": n_layers},
        "roofline": roof,
        "path_roofline": {"bytes": path_bytes, "flops": flops,
                          "hbm_GBps": round(path_bytes / (r["ms"] * 1e-3) / 1e9, 1),
                          "tflops": round(flops / (r["ms"] * 1e-3) / 1e12, 2)},
        "stage_us": {s: round(v * 1e3, 2) for s, v in r["stage_ms"].items()},
        "wall_ms_per_step": round(r["wall_ms"], 4),
    }
    if args.sweep:
        res["sweep"] = []
        for t in wl.tokens:
            rr = run_config(t, args.steps, args.warmup)
            res["sweep"].append({"tokens": t, "us_per_step": round(rr["ms"] * 1e3, 2),
                                 "tokens_per_s": round(t / (rr["ms"] * 1e-3), 1),
                                 "touched": rr["touched"],
                                 "stage_us": {s: round(v * 1e3, 2) for s, v in rr["stage_ms"].items()}})
    # plain copy of known size: reference reading for HBM byte counters
    src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        from oracle import formats, moe
        w, s, g, w_, s_, g_ = np_layers
        lay = moe.Layer(formats.Packed(fmt, w, s, g, 2 * I, H), formats.Packed(fmt, w_, s_, g_, H, I), k)
        res["cpu_baseline"] = cpu_baseline(lay, r["logits"], r["x"])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
