"""Seeded synthetic inputs for the MoE expert layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no quantization, routing or matmul).  Tests feed its float
weights to the CPU oracle's quantizers; the benchmark uses
:func:`random_packed`, which draws packed codes and scales directly.

Workloads mirror the Clef-Omni thinker's expert layer (hidden 2048, expert
intermediate 768, 128 experts, top-8).  The model cards measure on held-out
Clef records and benchmark suites that are not available here; these shapes
and distributions stand in for them:

* weights  N(0, 0.02) per expert matrix (then quantized by the caller);
* hidden   N(0, 1) rounded to bfloat16;
* logits   N(0, 1); optionally + a per-expert bias N(0, 0.5) (mild imbalance)
  or + ln p_e with p_r ~ r^-1.1 over ranks assigned by a seeded permutation
  (Zipf skew: a few experts receive most tokens).

Every stream is seeded by ``SeedSequence([workload_id, layer, tensor_id, ...])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

# tensor ids inside a SeedSequence key
_T_W13, _T_W2, _T_HIDDEN, _T_LOGITS, _T_BIAS, _T_PERM, _T_RESID = range(7)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    hidden: int
    inter: int
    experts: int
    top_k: int
    tokens: Tuple[int, ...]
    fmt: str                      # "int4_g128" | "fp8_b128" | "nvfp4_g16" | "stack"
    logits: str = "normal"        # "normal" | "bias" | "zipf"
    layers: int = 1
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(1, "tiny", 256, 128, 8, 2, (64,), "int4_g128",
                     notes="tiny layer, INT4 g128, CPU oracle in seconds"),
    "decode_int4": Workload(2, "decode_int4", 2048, 768, 128, 8, (1, 8, 64), "int4_g128",
                            notes="Clef-Omni-shaped decode layer, INT4 W4A16 g128"),
    "prefill_fp8": Workload(3, "prefill_fp8", 2048, 768, 128, 8, (4096,), "fp8_b128", "bias",
                            notes="prefill, FP8 E4M3 128x128 blocks, biased logits"),
    "nvfp4_zipf": Workload(4, "nvfp4_zipf", 2048, 768, 128, 8, (16384,), "nvfp4_g16", "zipf",
                           notes="NVFP4, Zipf(1.1)-skewed routing"),
    "stack48": Workload(5, "stack48", 2048, 768, 128, 8, (64, 2048), "stack", layers=48,
                        notes="48 layers: 0-23 FP8 128x128, 24-47 INT4 g128, residual chain"),
}


def stack_layer_format(layer: int) -> str:
    """Format of layer ``layer`` in the 48-layer stack (FP8 first, then INT4)."""
    return "fp8_b128" if layer < 24 else "int4_g128"


def rng(wid: int, layer: int, tensor: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wid, layer, tensor, *extra]))


def expert_weight(wid: int, layer: int, which: str, expert: int, n: int, k: int,
                  std: float = 0.02) -> np.ndarray:
    """Float32 [n, k] weights N(0, std) of one expert ('w13' or 'w2')."""
    t = _T_W13 if which == "w13" else _T_W2
    return (rng(wid, layer, t, expert).standard_normal((n, k), dtype=np.float32)
            * np.float32(std))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) and return the bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def hidden_bf16(wid: int, layer: int, tokens: int, hidden: int) -> np.ndarray:
    """bfloat16 bits [tokens, hidden] of N(0, 1) activations."""
    x = rng(wid, layer, _T_HIDDEN, tokens).standard_normal((tokens, hidden), dtype=np.float32)
    return to_bf16_bits(x)


def residual_bf16(wid: int, layer: int, tokens: int, hidden: int) -> np.ndarray:
    x = rng(wid, layer, _T_RESID, tokens).standard_normal((tokens, hidden), dtype=np.float32)
    return to_bf16_bits(x)


def router_logits(wid: int, layer: int, tokens: int, experts: int,
                  kind: str = "normal") -> np.ndarray:
    """Float32 router logits [tokens, experts]."""
    x = rng(wid, layer, _T_LOGITS, tokens).standard_normal((tokens, experts))
    if kind == "bias":
        x = x + rng(wid, layer, _T_BIAS).normal(0.0, 0.5, size=experts)[None, :]
    elif kind == "zipf":
        ranks = np.arange(1, experts + 1, dtype=np.float64)
        p = ranks ** -1.1
        p = p / p.sum()
        perm = rng(wid, layer, _T_PERM).permutation(experts)
        bias = np.empty(experts)
        bias[perm] = np.log(p)          # expert perm[r] gets rank r+1
        x = x + bias[None, :]
    elif kind != "normal":
        raise ValueError(kind)
    return x.astype(np.float32)


# INT4 codes are drawn from a rounded normal of this standard deviation: the
# code spread of N(0, 0.02) weights under a per-128 max-abs / 7 scale.
INT4_CODE_STD = 2.6


def random_packed(fmt: str, experts: int, n: int, k: int, seed: int):
    """Packed weights drawn directly, with the spread of quantized N(0, 0.02)
    weights: INT4 codes from a rounded normal, FP8 and E2M1 codes uniform, and
    scales of the magnitude such weights produce.  Returns (w, scale,
    gscale-or-None) numpy arrays in the library's layouts (see the header
    ``moe_quant.h``)."""
    g = np.random.default_rng(np.random.SeedSequence([seed, n, k]))
    if fmt == "int4_g128":
        q = np.clip(np.rint(g.standard_normal((experts, n, k), dtype=np.float32) * INT4_CODE_STD),
                    -8, 7).astype(np.uint8) + 8
        w = q[..., 0::2] | (q[..., 1::2] << 4)
        s = (0.02 * g.uniform(2.4, 3.4, size=(experts, n, k // 128)) / 7).astype(np.float16)
        return w, s, None
    if fmt == "fp8_b128":
        w = g.integers(0, 256, size=(experts, n, k), dtype=np.uint8)
        w[(w & 0x7F) == 0x7F] &= 0xF7        # no NaN codes
        s = (0.02 * g.uniform(4.0, 4.6, size=(experts, n // 128, k // 128)) / 448) \
            .astype(np.float32)
        return w, s, None
    if fmt == "nvfp4_g16":
        w = g.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
        s = g.integers(0x60, 0x7F, size=(experts, n, k // 16), dtype=np.uint8)
        gs = (448.0 * 6.0 / (0.02 * g.uniform(4.5, 5.5, size=experts))).astype(np.float32)
        return w, s, gs
    raise ValueError(fmt)


def random_packed_torch(fmt: str, experts: int, n: int, k: int, seed: int, device="cuda"):
    """Same recipe as :func:`random_packed`, drawn on the GPU with a seeded
    torch generator (for multi-layer stacks, where host generation is slow)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, n, k]).generate_state(1)[0]))
    u8 = dict(dtype=torch.uint8, device=device, generator=g)
    if fmt == "int4_g128":
        w = torch.empty((experts, n, k // 2), dtype=torch.uint8, device=device)
        for e in range(experts):        # one expert at a time bounds the float temporaries
            q = (torch.randn((n, k), device=device, generator=g) * INT4_CODE_STD).round_() \
                .clamp_(-8, 7).to(torch.int16) + 8
            w[e] = (q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8)
        s = (0.02 * (2.4 + torch.rand((experts, n, k // 128), device=device, generator=g)) / 7
             ).to(torch.float16)
        return w, s, None
    if fmt == "fp8_b128":
        w = torch.randint(0, 256, (experts, n, k), **u8)
        nan = (w & 0x7F) == 0x7F
        w[nan] = w[nan] & 0xF7
        s = (0.02 * (4.0 + 0.6 * torch.rand((experts, n // 128, k // 128), device=device,
                                             generator=g)) / 448).to(torch.float32)
        return w, s, None
    if fmt == "nvfp4_g16":
        w = torch.randint(0, 256, (experts, n, k // 2), **u8)
        s = torch.randint(0x60, 0x7F, (experts, n, k // 16), **u8)
        gs = (448.0 * 6.0 / (0.02 * (4.5 + torch.rand(experts, device=device, generator=g)))
              ).to(torch.float32)
        return w, s, gs
    raise ValueError(fmt)
