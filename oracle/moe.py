"""Routed MoE expert layer: routing, permutation, expert loop, combine (oracle).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

What the pages fix: the routed experts keep their weights packed and each
layer's experts are dequantized just in time for one grouped matmul
("clef-omni-fp8" card, section "How this checkpoint runs"; "clef-omni-int4"
card, section "How this checkpoint runs"; "clef-omni-NVFP4" card, section "How
it was made").  The router (mlp.gate) stays BF16 and unquantized
("clef-omni-int4" card, section "Recipe": ignore_layers=mlp.gate).  The gate
and up projections are stored concatenated, gate first ("clef-omni-NVFP4"
card, section "How it was made").

Readings taken where the pages are silent (all listed in the design doc):

* top-k by descending logit, ties to the lower expert id; weights are a
  softmax over the k selected logits (= softmax, top-k, renormalize);
* expert MLP: y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z);
* the layer output is the routing-weighted sum of the k expert outputs, added
  in slot order; an optional residual is added to it.

Everything is float64.  A grouped matmul over the same dequantized weights
reaches this result exactly up to rounding order, so the oracle is the plain
per-expert loop.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import formats


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), evaluated stably."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def router_logits(x_bf16_bits: np.ndarray, w_bf16_bits: np.ndarray) -> np.ndarray:
    """Router logits [T, E] of the gate that stays in BF16 ("clef-omni-fp8" card,
    section "What was quantized"; "clef-omni-NVFP4" card, section "How it was
    made", where the router mlp.gate is copied unchanged).

    Read as a linear layer without bias: logits[t, e] = sum_h x[t, h] w[e, h],
    with ``x`` the BF16 hidden rows [T, H] and ``w`` the gate's BF16 weight
    [E, H] (bit patterns).  BF16 values widen exactly to float64; each product
    is exact there and the sum rounds in float64.
    """
    x = bf16_bits_to_f64(x_bf16_bits)
    w = bf16_bits_to_f64(w_bf16_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("need x [T, H] and w [E, H]")
    return x @ w.T


def route(logits: np.ndarray, k: int):
    """Top-k expert selection and routing weights for each token.

    ``logits`` [T, E] are the router outputs (float32, or bfloat16 already
    widened; the values are compared exactly).  Returns ``ids`` int32 [T, k]
    ordered by descending logit with ties to the lower expert id, and ``w``
    float64 [T, k] = softmax over the k selected logits.
    """
    logits = np.asarray(logits, dtype=np.float64)
    t, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((t, k), dtype=np.int32)
    for i in range(t):
        # stable lexicographic order on (-logit, expert id)
        order = sorted(range(e), key=lambda j: (-logits[i, j], j))
        ids[i] = order[:k]
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    p = np.exp(sel - m)
    w = p / p.sum(axis=1, keepdims=True)
    return ids, w


@dataclass
class Permutation:
    counts: np.ndarray            # int32 [E]
    offsets: np.ndarray           # int32 [E+1], exclusive prefix sum of counts
    sorted_token_ids: np.ndarray  # int32 [T*k]: token of each grouped row
    sorted_slots: np.ndarray      # int32 [T*k]: flat slot t*k + j of each row
    inv_pos: np.ndarray           # int32 [T*k]: grouped row of slot t*k + j


def permute(ids: np.ndarray, num_experts: int) -> Permutation:
    """Group the T*k (token, slot) pairs by expert, stably by token.

    Counting sort: rows of expert 0 first, then expert 1, ...; inside one
    expert rows are in ascending token order (a token reaches an expert at most
    once, so this order is total).
    """
    ids = np.asarray(ids)
    t, k = ids.shape
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in ids.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    sorted_tok = np.empty(t * k, dtype=np.int32)
    sorted_slot = np.empty(t * k, dtype=np.int32)
    inv = np.empty(t * k, dtype=np.int32)
    for tok in range(t):
        for j in range(k):
            e = ids[tok, j]
            r = cursor[e]
            cursor[e] += 1
            sorted_tok[r] = tok
            sorted_slot[r] = tok * k + j
            inv[tok * k + j] = r
    return Permutation(counts.astype(np.int32), offsets.astype(np.int32),
                       sorted_tok, sorted_slot, inv)


def expert_mlp(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on rows x [n, H]; w13 [2I, H] (gate rows first), w2 [H, I]."""
    i = w13.shape[0] // 2
    gu = x @ w13.T
    gate, up = gu[:, :i], gu[:, i:]
    h = silu(gate) * up
    return h @ w2.T


@dataclass
class Layer:
    """One MoE expert layer in a packed format."""

    w13: formats.Packed   # [E, 2I, H]
    w2: formats.Packed    # [E, H, I]
    top_k: int

    @property
    def num_experts(self) -> int:
        return self.w13.num_experts

    @property
    def hidden(self) -> int:
        return self.w13.k

    @property
    def intermediate(self) -> int:
        return self.w13.n // 2


def moe_forward(layer: Layer, logits: np.ndarray, x_bf16_bits: np.ndarray,
                residual_bf16_bits: Optional[np.ndarray] = None,
                tokens: Optional[np.ndarray] = None):
    """Float64 layer output y [T, H] (plus the residual if one is given).

    ``tokens`` restricts the evaluation to a subset of token indices (the
    routing of a token depends only on its own logits, so the rows returned
    are exactly those of the full evaluation).  Returns (y, ids, w).
    """
    logits = np.asarray(logits)
    t_all = logits.shape[0]
    if tokens is None:
        tokens = np.arange(t_all)
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w = route(logits[tokens], layer.top_k)
    x = bf16_bits_to_f64(np.asarray(x_bf16_bits)[tokens])
    perm = permute(ids, layer.num_experts)
    # per-expert FP64 loop over the dequantized weights
    expert_out = np.empty((len(tokens) * layer.top_k, layer.hidden), dtype=np.float64)
    for e in range(layer.num_experts):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi == lo:
            continue
        rows = perm.sorted_token_ids[lo:hi]
        w13 = formats.dequantize_expert(layer.w13, e)
        w2 = formats.dequantize_expert(layer.w2, e)
        expert_out[lo:hi] = expert_mlp(x[rows], w13, w2)
    y = combine(perm, w, expert_out)
    if residual_bf16_bits is not None:
        y = y + bf16_bits_to_f64(np.asarray(residual_bf16_bits)[tokens])
    return y, ids, w


def combine(perm: Permutation, w: np.ndarray, expert_out: np.ndarray) -> np.ndarray:
    """Routing-weighted sum of the k expert outputs of every token, in slot order.

    ``expert_out`` [T*k, H] holds the expert outputs in grouped row order (row
    ``perm.inv_pos[t*k + j]`` is slot j of token t); ``w`` [T, k] the routing
    weights.  Returns y [T, H] = sum_j w[t, j] * expert_out[row(t, j)].
    """
    t, k = w.shape
    y = np.zeros((t, expert_out.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = perm.inv_pos[np.arange(t) * k + j]
        y += w[:, j:j + 1] * expert_out[rows]
    return y
