"""Seeded synthetic inputs for the fine-grained FP8 linear path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no absmax, scale, cast or GEMM), so both the GPU tests and
the CPU oracle can be fed from it.  Every tensor is drawn in float32 (or
float64 for Student-t) with ``numpy.random.default_rng([0, workload, tensor])``
and rounded once to bfloat16 (round-to-nearest-even, torch's CPU cast).
Results are returned as bfloat16 bit patterns (``uint16``).

The shapes and value distributions are those of the five workloads of the
method's hot path:

1. ``fprop_small``: Fprop only, X [256, 512] ~ N(0, 1) with exactly 131
   (0.1 %) positions multiplied by 50, W [512, 256] ~ N(0, 0.02).
2. ``linear_dsv3_attn``: one linear forward + backward at the DeepSeek-V3
   attention-projection shape: X [4096, 7168], W [7168, 7168] ~ N(0, 0.02),
   dY [4096, 7168] ~ N(0, 1e-3).
3. ``ffn_dense``: the dense FFN, up X [8192, 7168] ~ Student-t(3),
   W_up [7168, 18432] ~ N(0, 0.02), dY_up [8192, 18432] ~ N(0, 1e-3); down
   H [8192, 18432] ~ Student-t(3), W_down [18432, 7168], dY_down [8192, 7168].
4. ``moe_grouped``: one GPU's expert share: 32 experts, 8192 tokens routed to
   8 distinct experts each by Gumbel-top-8 over Zipf(1.1) popularities with 3
   experts forced empty; rows grouped per expert in 128-aligned, zero-padded
   segments.  W_gate/up [32, 7168, 4096], W_down [32, 2048, 7168].
5. ``quant_stress``: [16384, 7168] with per-row scales 10^U(-6, 3), 1 %
   scattered +-0, whole zero tiles in the 1x128, 128x1 and 128x128 tilings,
   1 % tiny negatives that quantize to -0, and a few bf16-subnormal negatives.
"""
from __future__ import annotations

import numpy as np
import torch

TILE = 128

WORKLOADS = {
    1: "fprop_small",
    2: "linear_dsv3_attn",
    3: "ffn_dense",
    4: "moe_grouped",
    5: "quant_stress",
}


def rng(workload: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([0, workload, tensor])


def bf16_bits(a) -> np.ndarray:
    """float32/float64 array -> bfloat16 bit patterns (uint16), RNE via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std: float, workload: int, tensor: int) -> np.ndarray:
    g = rng(workload, tensor)
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return bf16_bits(a)


def student_t_bf16(shape, nu: float, workload: int, tensor: int) -> np.ndarray:
    g = rng(workload, tensor)
    return bf16_bits(g.standard_t(nu, size=shape).astype(np.float32))


# ---------------------------------------------------------------------------
# Workload 1: Fprop only
# ---------------------------------------------------------------------------

def fprop_small():
    M, K, N = 256, 512, 256
    g = rng(1, 0)
    x = g.standard_normal(size=(M, K), dtype=np.float32)
    n_out = int(round(0.001 * M * K))  # 131
    pos = g.choice(M * K, size=n_out, replace=False)
    x.reshape(-1)[pos] *= np.float32(50.0)
    w = rng(1, 1).standard_normal(size=(K, N), dtype=np.float32) * np.float32(0.02)
    return {"x": bf16_bits(x), "w": bf16_bits(w), "M": M, "K": K, "N": N}


# ---------------------------------------------------------------------------
# Workload 2: linear fwd + bwd at the DSv3 attention-projection shape
# ---------------------------------------------------------------------------

def linear_dsv3_attn(M: int = 4096, K: int = 7168, N: int = 7168):
    return {
        "x": normal_bf16((M, K), 0.02, 2, 0),
        "w": normal_bf16((K, N), 0.02, 2, 1),
        "dy": normal_bf16((M, N), 1e-3, 2, 2),
        "M": M, "K": K, "N": N,
    }


# ---------------------------------------------------------------------------
# Workload 3: dense FFN (up and down projections)
# ---------------------------------------------------------------------------

def ffn_dense_up(M: int = 8192, K: int = 7168, N: int = 18432):
    return {
        "x": student_t_bf16((M, K), 3.0, 3, 0),
        "w": normal_bf16((K, N), 0.02, 3, 1),
        "dy": normal_bf16((M, N), 1e-3, 3, 2),
        "M": M, "K": K, "N": N,
    }


def ffn_dense_down(M: int = 8192, K: int = 18432, N: int = 7168):
    return {
        "x": student_t_bf16((M, K), 3.0, 3, 3),
        "w": normal_bf16((K, N), 0.02, 3, 4),
        "dy": normal_bf16((M, N), 1e-3, 3, 5),
        "M": M, "K": K, "N": N,
    }


# ---------------------------------------------------------------------------
# Workload 4: grouped MoE experts
# ---------------------------------------------------------------------------

def moe_routing(tokens: int = 8192, experts: int = 32, topk: int = 8,
                n_empty: int = 3, zipf_a: float = 1.1, workload: int = 4):
    """Per-token Gumbel-top-k over log popularities w_e = rank_e^-a.

    Ranks are a seeded permutation of 1..E; ``n_empty`` experts get w = 0 and
    so receive no token.  Returns (choice [tokens, topk] int64, loads [E]).
    """
    g = rng(workload, 100)
    ranks = g.permutation(experts) + 1
    logw = -zipf_a * np.log(ranks.astype(np.float64))
    empty = g.choice(experts, size=n_empty, replace=False)
    logw[empty] = -np.inf
    gumbel = -np.log(-np.log(g.random(size=(tokens, experts))))
    keys = logw[None, :] + gumbel
    choice = np.argsort(-keys, axis=1, kind="stable")[:, :topk]
    loads = np.bincount(choice.reshape(-1), minlength=experts)
    return choice, loads


def moe_layout(loads, align: int = TILE):
    """Expert-major row layout: segment e holds loads[e] rows padded to ``align``."""
    loads = np.asarray(loads, dtype=np.int64)
    padded = -(-loads // align) * align
    offsets = np.zeros(loads.size + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    return offsets


def moe_grouped(tokens: int = 8192, experts: int = 32, topk: int = 8, d_model: int = 7168,
                d_ff2: int = 4096, d_ff: int = 2048, with_weights: bool = True):
    """Grouped operands for the expert gate/up (d_model -> 2*d_ff) and down
    (d_ff -> d_model) projections.  Padding rows are zero."""
    choice, loads = moe_routing(tokens, experts, topk)
    offsets = moe_layout(loads)
    R_pad = int(offsets[-1])
    xt = normal_bf16((tokens, d_model), 1.0, 4, 0)
    # rows of expert e, in token order
    tok_of_slot = np.repeat(np.arange(tokens), topk)
    exp_of_slot = choice.reshape(-1)
    order = np.lexsort((tok_of_slot, exp_of_slot))
    row_token = np.full(R_pad, -1, dtype=np.int64)
    valid = np.zeros(R_pad, dtype=bool)
    sorted_exp = exp_of_slot[order]
    sorted_tok = tok_of_slot[order]
    for e in range(experts):
        sel = sorted_tok[sorted_exp == e]
        a = int(offsets[e])
        row_token[a:a + sel.size] = sel
        valid[a:a + sel.size] = True
    xg = np.zeros((R_pad, d_model), dtype=np.uint16)
    xg[valid] = xt[row_token[valid]]

    def rows_normal(width, std, tensor):
        out = np.zeros((R_pad, width), dtype=np.uint16)
        out[valid] = normal_bf16((int(valid.sum()), width), std, 4, tensor)
        return out

    d = {
        "offsets": offsets, "loads": loads, "valid": valid, "R_pad": R_pad,
        "x": xg,
        "h": rows_normal(d_ff, 1.0, 1),
        "dy_up": rows_normal(d_ff2, 1e-3, 2),
        "dy_down": rows_normal(d_model, 1e-3, 3),
        "E": experts, "d_model": d_model, "d_ff2": d_ff2, "d_ff": d_ff,
    }
    if with_weights:
        d["w_up"] = np.stack([normal_bf16((d_model, d_ff2), 0.02, 4, 10 + e) for e in range(experts)])
        d["w_down"] = np.stack([normal_bf16((d_ff, d_model), 0.02, 4, 100 + e) for e in range(experts)])
    return d


# ---------------------------------------------------------------------------
# Workload 5: quantization stress
# ---------------------------------------------------------------------------

def quant_stress(R: int = 16384, C: int = 7168, workload: int = 5):
    g = rng(workload, 0)
    sigma = np.power(10.0, g.uniform(-6.0, 3.0, size=(R, 1))).astype(np.float32)
    x = g.standard_normal(size=(R, C), dtype=np.float32)
    x *= sigma
    n = R * C
    flat = x.reshape(-1)
    # 1 % scattered exact zeros of both signs
    z = g.choice(n, size=n // 100, replace=False)
    flat[z] = np.where(g.random(z.size) < 0.5, np.float32(0.0), np.float32(-0.0))
    # 1 % scattered tiny negatives, far below half an E4M3 step of their tile
    tneg = g.choice(n, size=n // 100, replace=False)
    rows_of = tneg // C
    flat[tneg] = -sigma[rows_of, 0] * np.float32(1e-7)
    # whole zero tiles (random zero signs) in each tiling
    def signed_zeros(shape):
        return np.where(g.random(shape) < 0.5, np.float32(0.0), np.float32(-0.0))
    nb_c, nb_r = -(-C // TILE), -(-R // TILE)
    for r, j in zip(g.integers(0, R, 64), g.integers(0, nb_c, 64)):        # 1x128 segments
        seg = x[r, j * TILE:(j + 1) * TILE]
        seg[...] = signed_zeros(seg.shape)
    for i, c in zip(g.integers(0, nb_r, 64), g.integers(0, C, 64)):        # 128x1 column runs
        col = x[i * TILE:(i + 1) * TILE, c]
        col[...] = signed_zeros(col.shape)
    for i, j in zip(g.integers(0, nb_r, 8), g.integers(0, nb_c, 8)):        # 128x128 blocks
        blk = x[i * TILE:(i + 1) * TILE, j * TILE:(j + 1) * TILE]
        blk[...] = signed_zeros(blk.shape)
    bits = bf16_bits(x)
    # a few bf16-subnormal negatives (exponent field 0, nonzero mantissa)
    sub = g.choice(n, size=256, replace=False)
    bits.reshape(-1)[sub] = (0x8000 | g.integers(1, 0x80, sub.size)).astype(np.uint16)
    return {"x": bits, "R": R, "C": C}
