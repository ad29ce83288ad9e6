"""Shared helpers of the GPU parity tests: build packed layers (oracle
quantizer or directly drawn codes), run the HIP path through the C ABI, and
compare against the oracle."""
from __future__ import annotations

import multiprocessing
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import formats, moe
from weight_quantized_moe_amd import synth

RTOL_L2 = 2e-3      # max relative L2 error of a layer output vs the float64 oracle
ATOL_MAX = 2e-2     # max absolute error


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _quant_one(args):
    fmt, wid, layer, which, e, n, k = args
    w = synth.expert_weight(wid, layer, which, e, n, k).astype(np.float64)
    return formats.quantize_expert(fmt, w)


def quantized_layer(fmt, wid, layer, E, H, I, workers=None):
    """Oracle-quantized N(0, 0.02) weights of one layer (Packed w13, Packed w2)."""
    out = []
    for which, n, k in (("w13", 2 * I, H), ("w2", H, I)):
        p = formats.empty_packed(fmt, E, n, k)
        jobs = [(fmt, wid, layer, which, e, n, k) for e in range(E)]
        if E * n * k > 4_000_000:
            nproc = workers or min(16, len(os.sched_getaffinity(0)))
            ctx = multiprocessing.get_context("spawn")
            with ProcessPoolExecutor(nproc, mp_context=ctx) as ex:
                res = list(ex.map(_quant_one, jobs, chunksize=4))
        else:
            res = [_quant_one(j) for j in jobs]
        for e, (pw, s, g) in enumerate(res):
            p.w[e] = pw
            p.scale[e] = s
            if g is not None:
                p.gscale[e] = g
        out.append(p)
    return out[0], out[1]


def quantize_expert_job(args):
    """Worker job: oracle-quantized N(0, 0.02) weights of one expert of one
    layer.  Returns ((w, scale, gscale) of w13, (w, scale, gscale) of w2)."""
    fmt, wid, layer, e, H, I = args
    out = []
    for which, n, k in (("w13", 2 * I, H), ("w2", H, I)):
        w = synth.expert_weight(wid, layer, which, e, n, k).astype(np.float64)
        out.append(formats.quantize_expert(fmt, w))
    return tuple(out)


def expert_outputs_job(args):
    """Worker job: the oracle's SwiGLU expert (float64, exact dequantization)
    on each of several row sets.  ``q`` is quantize_expert_job's result;
    ``row_sets`` a list of float64 [n, H] arrays (or None)."""
    fmt, H, I, q, row_sets = args
    (w13, s13, g13), (w2, s2, g2) = q
    one = lambda a: None if a is None else np.asarray(a)[None]  # noqa: E731
    p13 = formats.Packed(fmt, one(w13), one(s13), one(g13), 2 * I, H)
    p2 = formats.Packed(fmt, one(w2), one(s2), one(g2), H, I)
    d13 = formats.dequantize_expert(p13, 0)
    d2 = formats.dequantize_expert(p2, 0)
    return [None if x is None or len(x) == 0 else moe.expert_mlp(x, d13, d2) for x in row_sets]


def oracle_forward_pool(pool, p13, p2, top_k, logits, x_bits):
    """The oracle's layer output for every token, with the per-expert step
    (dequantize + SwiGLU expert, float64) farmed to ``pool``: route, permute
    and combine are the oracle's own functions, in the order moe_forward runs
    them, so the result equals moe.moe_forward's (checked on the CPU)."""
    fmt, H, I, E = p13.fmt, p13.k, p13.n // 2, p13.num_experts
    ids, w = moe.route(logits, top_k)
    perm = moe.permute(ids, E)
    x = moe.bf16_bits_to_f64(x_bits)
    g = lambda p, e: None if p.gscale is None else p.gscale[e]  # noqa: E731
    futs = {}
    for e in range(E):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            q = ((p13.w[e], p13.scale[e], g(p13, e)), (p2.w[e], p2.scale[e], g(p2, e)))
            futs[e] = pool.submit(expert_outputs_job,
                                  (fmt, H, I, q, [x[perm.sorted_token_ids[lo:hi]]]))
    expert_out = np.empty((len(ids) * top_k, H), dtype=np.float64)
    for e, f in futs.items():
        expert_out[perm.offsets[e]:perm.offsets[e + 1]] = f.result()[0]
    return moe.combine(perm, w, expert_out), ids, w


def w4a4_expert_job(args):
    """Worker job: the W4A4 oracle's expert step (oracle.w4a4.expert_w4a4) on
    one expert's quantized rows, plus the down projection of given
    intermediate values (teacher forcing).  Returns (expert output, h in
    FP32, forced output)."""
    from oracle import w4a4
    H, I, q, xq, g_h, h_forced = args
    (w13, s13, g13), (w2, s2, g2) = q
    p13 = formats.Packed(formats.NVFP4, np.asarray(w13)[None], np.asarray(s13)[None], np.asarray(g13)[None], 2 * I, H)
    p2 = formats.Packed(formats.NVFP4, np.asarray(w2)[None], np.asarray(s2)[None], np.asarray(g2)[None], H, I)
    d13 = formats.dequantize_expert(p13, 0)
    d2 = formats.dequantize_expert(p2, 0)
    y, h32 = w4a4.expert_w4a4(xq, d13, d2, g_h)
    return y, h32, (None if h_forced is None else h_forced @ d2.T)


def oracle_w4a4_pool(pool, p13, p2, top_k, logits, x_bits, g_x, g_h, h_forced=None):
    """oracle.w4a4.moe_forward_w4a4 for every token with the per-expert step
    farmed to ``pool`` (route, permute, activation quantization and combine
    are the oracle's own functions, in its order), plus, if ``h_forced``
    (float64 [T*k, I], grouped order) is given, the teacher-forced output
    oracle.w4a4.down_from_values would give.  Returns (y, y_forced, h32)."""
    from oracle import w4a4
    H, I, E = p13.k, p13.n // 2, p13.num_experts
    ids, w = moe.route(logits, top_k)
    perm = moe.permute(ids, E)
    xq = w4a4.quantize_dequantize(moe.bf16_bits_to_f64(x_bits), g_x)
    futs = {}
    for e in range(E):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            q = ((p13.w[e], p13.scale[e], p13.gscale[e]), (p2.w[e], p2.scale[e], p2.gscale[e]))
            futs[e] = pool.submit(w4a4_expert_job, (H, I, q, xq[perm.sorted_token_ids[lo:hi]], g_h,
                                                    None if h_forced is None else h_forced[lo:hi]))
    R = len(ids) * top_k
    out = np.empty((R, H))
    forced = np.empty((R, H)) if h_forced is not None else None
    h32 = np.empty((R, I), np.float32)
    for e, f in futs.items():
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        y, h, yf = f.result()
        out[lo:hi], h32[lo:hi] = y, h
        if forced is not None:
            forced[lo:hi] = yf
    return (moe.combine(perm, w, out), None if forced is None else moe.combine(perm, w, forced), h32)


def _single_threaded_blas():
    """Pool initializer: one BLAS thread per worker (the pool supplies the
    parallelism; nested BLAS threads would oversubscribe the cores)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def spawn_pool(workers=None):
    nproc = workers or min(16, len(os.sched_getaffinity(0)))
    return ProcessPoolExecutor(nproc, mp_context=multiprocessing.get_context("spawn"),
                               initializer=_single_threaded_blas)


def random_layer(fmt, seed, E, H, I):
    """Packed weights drawn directly (codes and scales with the spread of
    quantized N(0, 0.02) weights)."""
    w, s, g = synth.random_packed(fmt, E, 2 * I, H, seed)
    p13 = formats.Packed(fmt, w, s, g, 2 * I, H)
    w, s, g = synth.random_packed(fmt, E, H, I, seed + 1)
    p2 = formats.Packed(fmt, w, s, g, H, I)
    return p13, p2


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class GpuLayer:
    def __init__(self, p13, p2, top_k):
        from weight_quantized_moe_amd import Layer
        self.p13, self.p2, self.top_k = p13, p2, top_k
        self.t = [dev(p13.w), dev(p13.scale), dev(p2.w), dev(p2.scale)]
        g13 = dev(p13.gscale) if p13.gscale is not None else None
        g2 = dev(p2.gscale) if p2.gscale is not None else None
        self.t += [g13, g2]
        self.layer = Layer(p13.fmt, self.t[0], self.t[1], self.t[2], self.t[3], top_k,
                           w13_gscale=g13, w2_gscale=g2)
        self.oracle = moe.Layer(p13, p2, top_k)

    def run(self, logits, x_bits, res_bits=None, probe=False, logits_bf16=False):
        import torch
        T = x_bits.shape[0]
        E, k, I = self.layer.num_experts, self.top_k, self.layer.inter
        lg = dev(logits)
        if logits_bf16:
            lg = lg.view(torch.bfloat16)
        x = dev(x_bits.view(np.int16)).view(torch.bfloat16)
        res = dev(res_bits.view(np.int16)).view(torch.bfloat16) if res_bits is not None else None
        pr = None
        if probe:
            pr = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                      topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                      expert_offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                      sorted_token_ids=torch.empty(T * k, dtype=torch.int32, device="cuda"),
                      inv_pos=torch.empty(T * k, dtype=torch.int32, device="cuda"),
                      h=torch.empty((T * k, I), dtype=torch.float16, device="cuda"))
        ws = self.layer.workspace(T)
        out = self.layer.forward(lg, x, residual=res, workspace=ws, probe=pr)
        torch.cuda.synchronize()
        out_np = out.view(torch.int16).cpu().numpy().view(np.uint16)
        pr_np = {k_: v.cpu().numpy() for k_, v in pr.items()} if pr else None
        overflow = self.layer.check(ws)
        return out_np, pr_np, overflow


def errors(out_bits, y_ref):
    y = moe.bf16_bits_to_f64(out_bits)
    rel = float(np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    mx = float(np.abs(y - y_ref).max()) if y.size else 0.0
    if y.size and mx > ATOL_MAX:
        i = np.unravel_index(np.argmax(np.abs(y - y_ref)), y.shape)
        ulp = 2.0 ** (np.floor(np.log2(max(abs(y_ref[i]), 2.0 ** -126))) - 7)
        log(f"    worst element {tuple(int(v) for v in i)}: got {y[i]!r} oracle {y_ref[i]!r} "
            f"(= {abs(y[i] - y_ref[i]) / ulp:.2f} bf16 ulp); output rms "
            f"{float(np.sqrt(np.mean(y_ref ** 2))):.4g}, max {float(np.abs(y_ref).max()):.4g}")
    return rel, mx


def check_routing(pr, logits, k, E):
    """Bit-exact routing and grouping against the oracle."""
    ids, w = moe.route(logits, k)
    assert np.array_equal(pr["topk_ids"], ids), "top-k ids differ"
    assert np.allclose(pr["topk_w"], w, rtol=2e-6, atol=1e-7), "routing weights differ"
    p = moe.permute(ids, E)
    assert np.array_equal(pr["expert_offsets"], p.offsets), "expert offsets differ"
    assert np.array_equal(pr["sorted_token_ids"], p.sorted_token_ids), "grouped token order differs"
    assert np.array_equal(pr["inv_pos"], p.inv_pos), "inverse positions differ"
