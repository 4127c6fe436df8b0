"""Shared helpers of the GPU parity tests (tolerances, seeded operands).

GEMM tolerance.  The stated bar for the block-scaled GEMM is
|C - C_ref| <= 1e-5 * (|A||B|)_ij (FP32 accumulation), plus one BF16 ulp of
C_ref for BF16 output.  That bar assumes every product reaches an FP32
accumulator intact.  gfx950's FP8 matrix cores do not do that (measured with
in-bounds probes of v_mfma_scale_f32_32x32x64_f8f6f4 and the other FP8 MFMA
forms): the products of each run of 8 consecutive K elements held by one
lane are summed in a fixed-point window aligned to the run's largest product
2^E_G, and every product bit below 2^(E_G - 13) is dropped (toward zero).
A product of two E4M3 values has at most 8 significant bits, so products
with |p| >= 2^(E_G - 6) are exact and any other loses less than
min(|p|, 2^(E_G - 13)).  The kernel feeds each lane aligned 8-runs of K, so
the derived bound adds, per output,
    H_ij = sum over aligned 8-runs G of K, over p in G with |p| < 2^(E_G-6),
           of min(|p|, 2^(E_G - 13))
to the stated one.  H_ij is zero whenever every run's products lie within 2^6
of each other; it is large only for runs where an outlier product dwarfs the
rest.  How many outputs also meet the stated bar is reported separately.
"""
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


def window_bound_pairs(deq_a: np.ndarray, deq_b: np.ndarray) -> np.ndarray:
    """H for paired rows: deq_a[e] . deq_b[e] (both [n, K] float64) -> [n]."""
    n, K = deq_a.shape
    p = np.abs(deq_a * deq_b).reshape(n, K // 8, 8)
    m = p.max(axis=2, keepdims=True)
    E = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    lsb = np.ldexp(1.0, (E - 13).astype(int))
    exact = p >= np.ldexp(1.0, (E - 6).astype(int))
    c = np.where(exact | (m == 0), 0.0, np.minimum(p, lsb))
    return c.sum(axis=(1, 2))


def window_bound_full(deq_a: np.ndarray, deq_b: np.ndarray, rows_per_chunk: int = 8) -> np.ndarray:
    """H for every output of deq_a [M, K] x deq_b [N, K]^T -> [M, N]."""
    M, K = deq_a.shape
    N = deq_b.shape[0]
    out = np.zeros((M, N))
    for i0 in range(0, M, rows_per_chunk):
        a = deq_a[i0:i0 + rows_per_chunk]
        c = a.shape[0]
        p = np.abs(a[:, None, :] * deq_b[None, :, :]).reshape(c, N, K // 8, 8)
        m = p.max(axis=3, keepdims=True)
        E = np.floor(np.log2(np.where(m > 0, m, 1.0)))
        lsb = np.ldexp(1.0, (E - 13).astype(int))
        exact = p >= np.ldexp(1.0, (E - 6).astype(int))
        out[i0:i0 + c] = np.where(exact | (m == 0), 0.0, np.minimum(p, lsb)).sum(axis=(2, 3))
    return out


class GemmRef:
    """Oracle result of a block-scaled GEMM plus its tolerance terms."""

    def __init__(self, ref, bnd, hw):
        self.ref, self.bnd, self.hw = ref, bnd, hw


def gemm_ref(qa, sa, qb, sb) -> GemmRef:
    ref, bnd = oracle.gemm(qa, sa, qb, sb)
    hw = window_bound_full(oracle.dequantize_rowwise(qa, sa), oracle.dequantize_rowwise(qb, sb))
    return GemmRef(ref, bnd, hw)


def grouped_ref(off, qa, sa, qb, sb) -> GemmRef:
    ref, bnd = oracle.grouped_gemm(off, qa, sa, qb, sb)
    da = oracle.dequantize_rowwise(qa, sa)
    hw = np.zeros_like(ref)
    for g in range(qb.shape[0]):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            hw[lo:hi] = window_bound_full(da[lo:hi], oracle.dequantize_rowwise(qb[g], sb[g]))
    return GemmRef(ref, bnd, hw)


def assert_gemm_close(got: torch.Tensor, r: GemmRef, what: str = "") -> dict:
    """Check against the derived bound; return how the stated bar fared."""
    g = got.float().cpu().numpy().astype(np.float64)
    ref, bnd, hw = r.ref, r.bnd, r.hw
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    stated = 1e-5 * bnd
    if got.dtype == torch.bfloat16:
        stated = stated + ulp_bf16(ref)
    tol = stated + hw
    err = np.abs(g - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst ratio "
            f"{(err / np.maximum(tol, 1e-300)).max():.3g}; first "
            + ", ".join(f"({i},{j}) got {g[i, j]!r} ref {ref[i, j]!r} hw {hw[i, j]:.3g}"
                        for i, j in idx))
    zero = bnd == 0
    assert (g[zero] == 0).all(), f"{what}: nonzero output where every product is zero"
    return {"n": int(err.size), "within_stated": int((err <= stated).sum()),
            "max_err_over_bnd": float((err / np.where(bnd > 0, bnd, np.inf)).max())
            if err.size else 0.0}


def random_mx_operand(rng: np.random.Generator, rows: int, K: int, spread: int = 20):
    """A quantized operand [rows][K] as the hot path produces it: BF16 N(0,1)
    with 1% outliers x100, each 32-block scaled by a random power of two in
    [2^-spread, 2^spread] (so E8M0 codes cover a wide range), then quantized
    row-wise by the oracle.  Returns (E4M3 codes, E8M0 scales)."""
    x = rng.standard_normal((rows, K)).astype(np.float32)
    out = rng.random((rows, K)) < 0.01
    x[out] *= 100.0
    e = rng.integers(-spread, spread + 1, size=(rows, K // 32))
    x *= np.repeat(np.ldexp(1.0, e), 32, axis=1).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    return oracle.quantize_rowwise(mxsynth.bits(xb))


def full_range_codes(rng: np.random.Generator, rows: int, K: int, scale_lo=112, scale_hi=140):
    """Uniformly random finite E4M3 codes (every exponent, subnormals included)
    and random E8M0 scales: far wider in-block dynamic range than quantized
    data, used to exercise the hardware's internal summation."""
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

# ---------------------------------------------------------------------------
# full-size helpers: the oracle is single-threaded C called through ctypes
# (which releases the GIL), so large tensors are split over threads by rows.

def _pool_map(fn, items, workers=16):
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def oracle_rowwise_par(x_bits: np.ndarray, chunk: int = 256):
    rows = x_bits.shape[0]
    parts = _pool_map(lambda r0: oracle.quantize_rowwise(x_bits[r0:r0 + chunk]),
                      range(0, rows, chunk))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_colwise_par(x_bits: np.ndarray, chunk: int = 256):
    cols = x_bits.shape[1]
    parts = _pool_map(lambda c0: oracle.quantize_colwise(
        np.ascontiguousarray(x_bits[:, c0:c0 + chunk])), range(0, cols, chunk))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def sample_entries(rng, M: int, N: int, n: int = 2048):
    """Random (row, col) pairs plus the four corners and edges of C."""
    rows = rng.integers(0, M, size=n)
    cols = rng.integers(0, N, size=n)
    extra_r = np.array([0, 0, M - 1, M - 1] + list(range(min(M, 64))) + [M - 1] * min(N, 64))
    extra_c = np.array([0, N - 1, 0, N - 1] + [N - 1] * min(M, 64) + list(range(min(N, 64))))
    return np.concatenate([rows, extra_r]), np.concatenate([cols, extra_c])


def check_sampled(C: torch.Tensor, rows, cols, qa, sa, qb, sb, what: str) -> dict:
    """C[rows, cols] from the GPU against oracle entries of deq(A) deq(B)^T."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    ref, bnd = oracle.gemm_sampled(rows, cols, qa, sa, qb, sb)
    da = oracle.dequantize_rowwise(qa[rows], sa[rows])
    db = oracle.dequantize_rowwise(qb[cols], sb[cols])
    hw = window_bound_pairs(da, db)
    got = C[torch.from_numpy(rows).to(C.device), torch.from_numpy(cols).to(C.device)]
    r = GemmRef(ref[None, :], bnd[None, :], hw[None, :])
    return assert_gemm_close(got[None, :], r, what)


def check_sampled_grouped(C: torch.Tensor, rows, cols, off, qa, sa, qb, sb, what: str) -> dict:
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    ref, bnd = oracle.grouped_gemm_sampled(rows, cols, off, qa, sa, qb, sb)
    g = np.searchsorted(off, rows, side="right") - 1
    da = oracle.dequantize_rowwise(qa[rows], sa[rows])
    db = np.stack([oracle.dequantize_rowwise(qb[gi, c][None], sb[gi, c][None])[0]
                   for gi, c in zip(g, cols)])
    hw = window_bound_pairs(da, db)
    got = C[torch.from_numpy(rows).to(C.device), torch.from_numpy(cols).to(C.device)]
    r = GemmRef(ref[None, :], bnd[None, :], hw[None, :])
    return assert_gemm_close(got[None, :], r, what)
