"""The 48-layer stack: layers 0-23 FP8 128x128 block-scaled, 24-47 INT4 g128
(hidden 2048, expert intermediate 768, 128 experts, top-8), each layer's
weights N(0, 0.02) from its own seed and quantized by the oracle, router
logits N(0, 1) per layer, chained on the GPU with residual adds

    x_{l+1} = bf16(fp32(x_l) + y_l),   y_l = moe_l(x_l),

for a 64-token and a 2048-token batch at once.

Parity is per layer and teacher-forced: at every sixth layer and at both ends
of each format's range, the oracle runs that layer on the GPU's own BF16 input
x_l, and the GPU output y_l is compared on every token (rel-L2 over the whole
[T, H] output, max abs).  Beside it the test follows an FP32 chain (the
oracle's float64 layer outputs added without rounding) over all 64 tokens of
the small batch and 256 sampled tokens of the large one, and reports the
end-to-end drift of the GPU's BF16 residual stream from it: BF16 rounding of the
residual alone moves the stream by about 1e-2 after 48 layers, so the drift is
reported, and only checked against a loose bound that catches a broken chain.

The layers run in chunks of eight, one test each, over one module-level chain.
Quantization and the oracle's per-expert work run in a pool of spawned worker
processes (they never touch the GPU).
"""
import numpy as np
import pytest

from oracle import formats, moe
from weight_quantized_moe_amd import synth

from gpu_helpers import (ATOL_MAX, RTOL_L2, dev, errors, expert_outputs_job, log,
                         quantize_expert_job, spawn_pool)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["stack48"]
H, I, E, K, L = W.hidden, W.inter, W.experts, W.top_k, W.layers
CHECK = frozenset(range(0, L, 6)) | {23, 24, L - 1}
CHUNK = 8
DRIFT_SAMPLE = 256     # tokens of the 2048-token batch whose FP32 chain is followed
DRIFT_BOUND = 0.1      # sanity bound on the end-to-end drift (not a parity bar)


class _Chain:
    pass


@pytest.fixture(scope="module")
def chain():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_moe_amd import load_library
    load_library()
    c = _Chain()
    c.pool = spawn_pool()
    c.next = 0
    c.Ts = tuple(W.tokens)                      # (64, 2048)
    c.x = {}
    c.tok = {}
    c.x32 = {}
    rng = np.random.default_rng(20260)
    for T in c.Ts:
        x0 = synth.hidden_bf16(W.wid, 0, T, H)
        c.x[T] = dev(x0.view(np.int16)).view(torch.bfloat16)
        c.tok[T] = np.arange(T) if T <= 64 else np.sort(rng.choice(T, DRIFT_SAMPLE, replace=False))
        c.x32[T] = moe.bf16_bits_to_f64(x0)[c.tok[T]]
    c.quant = {}
    c.worst = 0.0
    yield c
    c.pool.shutdown()


def _submit_quant(c, layer):
    if layer < L and layer not in c.quant:
        fmt = synth.stack_layer_format(layer)
        c.quant[layer] = [c.pool.submit(quantize_expert_job, (fmt, W.wid, layer, e, H, I))
                          for e in range(E)]


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run_layer(c, layer):
    import torch
    from weight_quantized_moe_amd import Layer
    fmt = synth.stack_layer_format(layer)
    _submit_quant(c, layer)
    _submit_quant(c, layer + 1)             # keeps the pool busy while this layer finishes
    check = layer in CHECK
    lg = {T: synth.router_logits(W.wid, layer, T, E) for T in c.Ts}
    # row sets the oracle evaluates: the FP32 chains, and at checked layers
    # the GPU's own inputs (teacher forcing)
    sets = []
    for T in c.Ts:
        ids, w = moe.route(lg[T][c.tok[T]], K)
        sets.append((("fp32", T), w, moe.permute(ids, E), c.x32[T]))
        if check:
            ids, w = moe.route(lg[T], K)
            sets.append((("gpu", T), w, moe.permute(ids, E), moe.bf16_bits_to_f64(_bits(c.x[T]))))
    q = [f.result() for f in c.quant.pop(layer)]
    jobs = []
    for e in range(E):
        rows = []
        for _, _, perm, x in sets:
            lo, hi = perm.offsets[e], perm.offsets[e + 1]
            rows.append(x[perm.sorted_token_ids[lo:hi]] if hi > lo else None)
        jobs.append(c.pool.submit(expert_outputs_job, (fmt, H, I, q[e], rows)))

    # the GPU layer, from the same packed bytes
    p13 = formats.empty_packed(fmt, E, 2 * I, H)
    p2 = formats.empty_packed(fmt, E, H, I)
    for e, ((w13, s13, _), (w2, s2, _)) in enumerate(q):
        p13.w[e], p13.scale[e], p2.w[e], p2.scale[e] = w13, s13, w2, s2
    t = [dev(p13.w), dev(p13.scale), dev(p2.w), dev(p2.scale)]
    lay = Layer(fmt, t[0], t[1], t[2], t[3], K)
    y_gpu = {}
    for T in c.Ts:
        ws = lay.workspace(T)
        lgt = dev(lg[T])
        if check:
            y = lay.forward(lgt, c.x[T], workspace=ws)
            torch.cuda.synchronize()
            assert not lay.check(ws), f"layer {layer} T={T}: FP16 intermediate saturated"
            y_gpu[T] = _bits(y)
        c.x[T] = lay.forward(lgt, c.x[T], residual=c.x[T], workspace=ws)
    torch.cuda.synchronize()
    del lay, t

    outs = [j.result() for j in jobs]
    for si, (key, w, perm, x) in enumerate(sets):
        eo = np.zeros((int(perm.offsets[-1]), H), dtype=np.float64)
        for e in range(E):
            lo, hi = perm.offsets[e], perm.offsets[e + 1]
            if hi > lo:
                eo[lo:hi] = outs[e][si]
        y_ref = moe.combine(perm, w, eo)
        kind, T = key
        if kind == "fp32":
            c.x32[T] = c.x32[T] + y_ref
        else:
            rel, mx = errors(y_gpu[T], y_ref)
            c.worst = max(c.worst, rel)
            log(f"    layer {layer:2d} ({fmt}) T={T}: rel_l2={rel:.3e} max_abs={mx:.3e}")
            assert rel <= RTOL_L2 and mx <= ATOL_MAX, f"layer {layer} T={T}"


@pytest.mark.parametrize("chunk", range(L // CHUNK))
def test_stack48(chain, chunk):
    import torch
    first = chunk * CHUNK
    while chain.next < first:               # a chunk run alone first builds the chain up to it
        _run_layer(chain, chain.next)
        chain.next += 1
    log(f"[stack48] layers {first}-{first + CHUNK - 1}")
    for layer in range(first, first + CHUNK):
        _run_layer(chain, layer)
        chain.next = layer + 1
    for T in chain.Ts:
        xf = chain.x[T].float()
        assert torch.isfinite(xf).all()
        log(f"    after layer {chain.next - 1}: T={T} residual rms {xf.square().mean().sqrt().item():.4f}")
    if chain.next == L:
        log(f"    worst checked layer rel_l2={chain.worst:.3e}")
        for T in chain.Ts:
            got = moe.bf16_bits_to_f64(_bits(chain.x[T]))[chain.tok[T]]
            ref = chain.x32[T]
            drift = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
            log(f"    end-to-end drift vs the FP32 chain, T={T} ({len(chain.tok[T])} tokens): "
                f"rel_l2={drift:.3e}")
            assert drift <= DRIFT_BOUND
