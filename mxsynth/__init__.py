"""Seeded synthetic inputs for the MXFP8 hot path (shared by tests, smoke and bench).

This module holds no MXFP8 arithmetic: it only draws BF16 tensors with the
shapes and value structure of the workloads below and computes the per-expert
row counts of the MoE workload.  Both the HIP path and the CPU oracle take
their inputs from here; neither is imported by it.

Workloads follow the layer shapes of the two models measured in "End-to-End
MXFP8 Reinforcement Learning on Blackwell" (Table 2: Qwen3-8B dense, and
Qwen3-30B-A3B with 128 experts and top-8 routing; dynamic micro-batches of
12 288 and 20 480 tokens per GPU; Table 7: MXFP8 pays off above about 4.5k
tokens per micro-batch, hence M = 4608 for the dense forward).

Recipe: values are drawn in float32 on the CPU with ``torch.Generator``,
outlier and zero structure is applied, then the tensor is rounded to BF16
(round-to-nearest-even, torch's conversion).  N(0, s) means standard
deviation s.  Outlier positions are drawn without replacement from the same
generator, after the values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np
import torch

# ---------------------------------------------------------------------------
# primitive draws


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std: float, seed: int, outlier_frac: float = 0.0,
                outlier_mul: float = 1.0, device="cpu") -> torch.Tensor:
    """N(0, std) with a fraction of elements (chosen without replacement) multiplied.

    ``device`` picks where the generator runs: the CPU stream is the one the
    parity tests use; a device stream draws the same distribution faster but
    not the same numbers."""
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device) * std
    n = x.numel()
    k = int(round(outlier_frac * n))
    if k > 0:
        idx = torch.randperm(n, generator=g, device=device)[:k]
        x.view(-1)[idx] *= outlier_mul
    return x.to(torch.bfloat16)


def channel_outliers_bf16(rows: int, cols: int, std: float, seed: int, frac: float,
                          mul: float, device="cpu") -> torch.Tensor:
    """Activations N(0, std) whose ``frac`` of whole columns (channels) are multiplied."""
    g = _gen(seed, device)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32, device=device) * std
    k = int(round(frac * cols))
    if k > 0:
        ch = torch.randperm(cols, generator=g, device=device)[:k]
        x[:, ch] *= mul
    return x.to(torch.bfloat16)


def bits(x: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (a view of the same bytes)."""
    assert x.dtype == torch.bfloat16
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> BF16 tensor (CPU)."""
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16)


# ---------------------------------------------------------------------------
# MoE expert loads


def zipf_expert_rows(num_tokens: int = 20480, num_experts: int = 128, top_k: int = 8,
                     exponent: float = 1.1) -> np.ndarray:
    """Rows per expert after top-k routing with Zipf(exponent) popularity.

    Expert of rank r (1-based) gets a share proportional to r^-exponent of the
    num_tokens*top_k routed rows.  Routing picks distinct experts per token, so
    no expert can hold more than num_tokens rows: shares above that cap are
    clipped and the excess is water-filled over the remaining experts in the
    same proportions.  Integer counts use largest-remainder rounding.
    Expert e is rank e+1 (expert 0 is the most loaded)."""
    total = num_tokens * top_k
    w = np.arange(1, num_experts + 1, dtype=np.float64) ** (-exponent)
    share = np.zeros(num_experts)
    capped = np.zeros(num_experts, dtype=bool)
    for _ in range(num_experts):
        rest = total - num_tokens * capped.sum()
        free = ~capped
        share[free] = rest * w[free] / w[free].sum()
        share[capped] = num_tokens
        over = free & (share > num_tokens)
        if not over.any():
            break
        capped |= over
    base = np.floor(share).astype(np.int64)
    short = total - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:short]] += 1
    assert base.sum() == total and base.max() <= num_tokens
    return base


def offsets_from_rows(rows_per_group: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(rows_per_group)]).astype(np.int64)


# ---------------------------------------------------------------------------
# the five workloads


@dataclass
class GemmSpec:
    """C[M][N] = A[M][K] . B[N][K]^T with both operands K-contiguous."""
    name: str
    M: int
    N: int
    K: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# Qwen3-8B decoder-layer weights, [out][in] (row-major, K = in contiguous).
QWEN3_8B_WEIGHTS: List[Tuple[str, Tuple[int, int]]] = [
    ("q", (4096, 4096)), ("k", (1024, 4096)), ("v", (1024, 4096)), ("o", (4096, 4096)),
    ("gate", (12288, 4096)), ("up", (12288, 4096)), ("down", (4096, 12288)),
]

DENSE_FWD_TOKENS = 4608
DENSE_FWD_GEMMS = [GemmSpec("qkv", 4608, 6144, 4096), GemmSpec("o", 4608, 4096, 4096),
                   GemmSpec("gate_up", 4608, 24576, 4096), GemmSpec("down", 4608, 4096, 12288)]
DENSE_BWD_TOKENS = 12288
DENSE_BWD_GEMMS = [GemmSpec("dgrad", 12288, 4096, 24576), GemmSpec("wgrad", 24576, 4096, 12288)]
MOE_TOKENS, MOE_EXPERTS, MOE_TOPK, MOE_HIDDEN, MOE_FFN = 20480, 128, 8, 2048, 768


def tiny(seed: int = 0):
    """A[128x256], B[256x256] ~ N(0,1), 1% of elements x100, four all-zero 32-blocks each.

    A is row-wise quantized (blocks along its rows), B ([K][N]) column-wise
    (blocks down its columns).  Returns BF16 CPU tensors (A, B)."""
    g = _gen(seed)
    A = torch.randn(128, 256, generator=g, dtype=torch.float32)
    B = torch.randn(256, 256, generator=g, dtype=torch.float32)
    for X in (A, B):
        n = X.numel()
        idx = torch.randperm(n, generator=g)[: int(round(0.01 * n))]
        X.view(-1)[idx] *= 100.0
    # four distinct (row, 32-block) of A and (32-block, column) of B set to zero
    a_sel = torch.randperm(128 * 8, generator=g)[:4]
    for v in a_sel.tolist():
        r, kb = divmod(v, 8)
        A[r, 32 * kb:32 * kb + 32] = 0.0
    b_sel = torch.randperm(8 * 256, generator=g)[:4]
    for v in b_sel.tolist():
        kb, c = divmod(v, 256)
        B[32 * kb:32 * kb + 32, c] = 0.0
    return A.to(torch.bfloat16), B.to(torch.bfloat16)


def weight_sync(cfg_seed: int = 2000, device="cpu") -> Dict[str, torch.Tensor]:
    """One Qwen3-8B decoder layer's BF16 weights ~ N(0, 0.02), 0.1% of elements x20."""
    return {name: normal_bf16(shape, 0.02, cfg_seed + i, 0.001, 20.0, device)
            for i, (name, shape) in enumerate(QWEN3_8B_WEIGHTS)}


def dense_fwd_activations(seed: int = 3000, device="cpu"):
    """X_h[4608x4096] (input of qkv, o, gate_up) and X_i[4608x12288] (input of down),
    N(0,1) with 0.5% of channels x50."""
    xh = channel_outliers_bf16(DENSE_FWD_TOKENS, 4096, 1.0, seed, 0.005, 50.0, device)
    xi = channel_outliers_bf16(DENSE_FWD_TOKENS, 12288, 1.0, seed + 1, 0.005, 50.0, device)
    return xh, xi


def dense_fwd_weights(w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """Fused projections of the layer: qkv = [q; k; v], gate_up = [gate; up]."""
    return {"qkv": torch.cat([w["q"], w["k"], w["v"]], 0), "o": w["o"],
            "gate_up": torch.cat([w["gate"], w["up"]], 0), "down": w["down"]}


def dense_bwd_inputs(seed: int = 4000, device="cpu"):
    """dY[12288x24576] ~ N(0, 1e-3) (gradient of the gate_up output) and the
    layer input X[12288x4096] drawn like the forward activations."""
    dy = normal_bf16((DENSE_BWD_TOKENS, 24576), 1e-3, seed, device=device)
    x = channel_outliers_bf16(DENSE_BWD_TOKENS, 4096, 1.0, seed + 1, 0.005, 50.0, device)
    return dy, x


def moe_inputs(seed: int = 5000, device="cpu"):
    """Qwen3-30B-A3B MoE layer: routed rows sorted by expert.

    Returns (rows_per_expert[128], A_gu[163840x2048], A_dn[163840x768],
    W_gu[128][1536][2048], W_dn[128][2048][768]); activations N(0,1),
    weights N(0, 0.02)."""
    rows = zipf_expert_rows(MOE_TOKENS, MOE_EXPERTS, MOE_TOPK, 1.1)
    m = int(rows.sum())
    a_gu = normal_bf16((m, MOE_HIDDEN), 1.0, seed, device=device)
    a_dn = normal_bf16((m, MOE_FFN), 1.0, seed + 1, device=device)
    w_gu = normal_bf16((MOE_EXPERTS, 2 * MOE_FFN, MOE_HIDDEN), 0.02, seed + 2, device=device)
    w_dn = normal_bf16((MOE_EXPERTS, MOE_HIDDEN, MOE_FFN), 0.02, seed + 3, device=device)
    return rows, a_gu, a_dn, w_gu, w_dn


def moe_bwd_grads(seed: int = 5200, device="cpu"):
    """Gradients of the Qwen3-30B-A3B MoE layer's expert outputs, rows sorted by
    expert like moe_inputs: dY_gu[163840x1536] (gate_up output) and
    dY_dn[163840x2048] (down output), BF16 N(0, 1e-3) like the dense backward."""
    m = int(zipf_expert_rows(MOE_TOKENS, MOE_EXPERTS, MOE_TOPK, 1.1).sum())
    dy_gu = normal_bf16((m, 2 * MOE_FFN), 1e-3, seed, device=device)
    dy_dn = normal_bf16((m, MOE_HIDDEN), 1e-3, seed + 1, device=device)
    return dy_gu, dy_dn


WORKLOADS = {
    "tiny": "A[128x256] row-wise, B[256x256] column-wise, mx_gemm 128x256x256 BF16 out",
    "weight_sync": "row-wise + column-wise MXFP8 + scale rearrangement of one Qwen3-8B layer",
    "dense_fwd": "Qwen3-8B linears at M=4608: qkv, o, gate_up, down",
    "dense_bwd": "Qwen3-8B gate_up dgrad (12288x4096x24576) and wgrad (24576x4096x12288)",
    "moe": "Qwen3-30B-A3B grouped gate_up/down, 128 experts, top-8, Zipf(1.1) loads",
    "moe_bwd": "Qwen3-30B-A3B expert backward: per-expert dgrad (grouped over rows) and "
               "wgrad (grouped over each expert's token range) of gate_up and down",
}


def moe_routing(seed: int = 5100, num_tokens: int = MOE_TOKENS, num_experts: int = MOE_EXPERTS,
                top_k: int = MOE_TOPK, exponent: float = 1.1):
    """Top-k routing with the per-expert row counts of zipf_expert_rows.

    Returns (topk_ids int32 [num_tokens][top_k], weights float32 [num_tokens]
    [top_k]).  Expert e's rows[e] assignments go to distinct tokens (the
    experts' slots, laid out expert by expert, are dealt to tokens round-robin,
    and no expert holds more than num_tokens rows); tokens and the order of
    each token's experts are then shuffled.  Weights are positive and sum to
    1 per token (a softmax over seeded logits)."""
    rows = zipf_expert_rows(num_tokens, num_experts, top_k, exponent)
    flat = np.repeat(np.arange(num_experts, dtype=np.int32), rows)
    grid = np.empty((num_tokens, top_k), np.int32)
    i = np.arange(flat.size)
    grid[i % num_tokens, i // num_tokens] = flat
    rng = np.random.default_rng(seed)
    grid = grid[rng.permutation(num_tokens)]
    grid = np.take_along_axis(grid, np.argsort(rng.random(grid.shape), axis=1), axis=1)
    logits = rng.normal(0.0, 1.0, size=grid.shape)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return grid, w
