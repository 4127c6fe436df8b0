"""Shared helpers of the GPU parity tests (tolerances, seeded operands)."""
import numpy as np
import torch

import mxsynth
import oracle


def ulp_bf16(y: np.ndarray) -> np.ndarray:
    """One BF16 ulp at y: 2^(floor(log2|y|) - 7) for normal y, 2^-133 below."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    u = np.ldexp(1.0, (e - 7).astype(int))
    return np.where(a > 0, u, 2.0 ** -133)


def gemm_tolerance(ref: np.ndarray, bnd: np.ndarray, out_dtype) -> np.ndarray:
    """|C - C_ref| <= 1e-5 * (|A||B|)_ij, plus one BF16 ulp of C_ref for BF16 output."""
    tol = 1e-5 * bnd
    if out_dtype == torch.bfloat16:
        tol = tol + ulp_bf16(ref)
    return tol


def assert_gemm_close(got: torch.Tensor, ref: np.ndarray, bnd: np.ndarray, what: str = ""):
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    tol = gemm_tolerance(ref, bnd, got.dtype)
    err = np.abs(g - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst ratio "
            f"{(err / np.maximum(tol, 1e-300)).max():.3g}; first "
            + ", ".join(f"({i},{j}) got {g[i, j]!r} ref {ref[i, j]!r}" for i, j in idx))
    zero = bnd == 0
    assert (g[zero] == 0).all(), f"{what}: nonzero output where every product is zero"
    return float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0


def random_mx_operand(rng: np.random.Generator, rows: int, K: int, scale_lo=112, scale_hi=140):
    """Random finite E4M3 codes and E8M0 scales (a quantized operand [rows][K])."""
    q = rng.integers(0, 256, size=(rows, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38
    s = rng.integers(scale_lo, scale_hi, size=(rows, K // 32)).astype(np.uint8)
    return q, s


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(x: torch.Tensor, dev="cuda") -> torch.Tensor:
    return x.contiguous().to(dev)


def oracle_quant_rowwise(x: torch.Tensor):
    return oracle.quantize_rowwise(mxsynth.bits(x))


def oracle_quant_colwise(x: torch.Tensor):
    return oracle.quantize_colwise(mxsynth.bits(x))
