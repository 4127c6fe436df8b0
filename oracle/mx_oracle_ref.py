"""Second CPU oracle for MXFP8 quantization, scale rearrangement and the
block-scaled GEMM, written independently of oracle/mx_oracle.c.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): only tests/ use it, to
check the C oracle against a second implementation that takes a different
route to the same definitions.  It shares no code with the C oracle or with
the HIP library.

What it computes (the definitions the C oracle follows, reached otherwise):
  * MXFP8 quantization ("End-to-End MXFP8 Reinforcement Learning on
    Blackwell", Figure 1 and Table 6: BF16 tensors quantized to MXFP8 before
    every MXFP8 GEMM; Table 10, row F6: scales are E8M0, exponents only),
    with the OCP MX v1.0 shared-scale rule: per block of 32 elements,
    amax = max |v|, scale 2^(floor(log2 amax) - 8), every element divided by
    the scale and taken to the NEAREST finite E4M3 value, ties to the value
    whose mantissa is even, magnitudes past 448 clamped to 448.
    Here the nearest value is found by a search over the sorted table of all
    127 non-negative finite E4M3 values (the C oracle rounds by exponent and
    mantissa arithmetic instead), and floor(log2 amax) comes from numpy's
    frexp of the whole array.
  * Readings shared with the C oracle (each a reading of a silent page):
    all-zero block -> scale code 0; amax below 2^-119 -> scale code 0 (the
    clamp); NaN or Inf in a block -> scale code 0xFF and every element 0x7F;
    a negative value that rounds to zero keeps its sign (0x80); column-wise
    output transposed; the rearranged scale layout of 32-row x 8-block tiles
    (tile (rt, kt) at byte (rt*KT + kt)*256, entry (row 32rt + r, block
    8kt + 2t + h) at byte (32h + r)*4 + t, padding 0x7F).
  * The GEMM ("MXFP8 GEMMs", Figure 1; Table 6): C = deq(A) deq(B)^T with
    deq(q, c) = E4M3(q) * 2^(c - 127), by numpy's float64 matrix product, and
    the bound (|A||B|)_ij as the product of the magnitudes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

# ---- E4M3 ("E4M3FN") value table: code -> value, by the format definition
# (sign, 4 exponent bits of bias 7, 3 mantissa bits; exponent field 0 holds
# the subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN).


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256)
    for code in range(256):
        sign = -1.0 if code >= 128 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()
# the non-negative finite values in increasing order: codes 0x00 .. 0x7E
POS_CODES = np.arange(0x7F, dtype=np.uint8)
POS_VALUES = E4M3[:0x7F]
assert np.all(np.diff(POS_VALUES) > 0)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float64 (exact: BF16 is the top half of binary32)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_nearest(t: np.ndarray) -> np.ndarray:
    """Finite float64 array -> E4M3 codes: nearest finite value, ties to the
    code with an even mantissa, clamped at 448, sign of zero kept."""
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    hi = np.searchsorted(POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - POS_VALUES[lo]
    d_hi = POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (POS_CODES[hi] % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, POS_CODES[hi], POS_CODES[lo])
    code = np.where(a >= POS_VALUES[-1], POS_CODES[-1], code)      # at or past 448
    code = np.where(a <= POS_VALUES[lo], POS_CODES[lo], code)      # exact hits and a below 0x01
    neg = np.signbit(t)
    return (code | np.where(neg, 0x80, 0x00)).astype(np.uint8)


def quantize_rowwise(x_bits: np.ndarray):
    """BF16 bits [rows][cols] -> (codes [rows][cols], scales [rows][cols/32])."""
    x_bits = np.asarray(x_bits, np.uint16)
    rows, cols = x_bits.shape
    v = bf16_to_f64(x_bits).reshape(rows, cols // BLOCK, BLOCK)
    bad = ~np.isfinite(v).all(axis=2)
    amax = np.abs(np.where(np.isfinite(v), v, 0.0)).max(axis=2)
    _, e2 = np.frexp(amax)                      # amax = f * 2^e2 with f in [0.5, 1)
    floor_log2 = e2 - 1
    c = np.clip(floor_log2 - 8 + 127, 0, 254)
    c = np.where(amax == 0, 0, c)
    scale = np.ldexp(1.0, (c - 127).astype(np.int64))
    t = np.where(np.isfinite(v), v, 0.0) / scale[..., None]
    q = e4m3_nearest(t)
    q = np.where(bad[..., None], np.uint8(0x7F), q)
    c = np.where(bad, 255, c)
    return q.reshape(rows, cols).astype(np.uint8), c.astype(np.uint8)


def quantize_colwise(x_bits: np.ndarray):
    """Column-wise blocks, output transposed: colwise(X) is rowwise(X^T)."""
    return quantize_rowwise(np.ascontiguousarray(np.asarray(x_bits, np.uint16).T))


def scale_swizzle(s: np.ndarray) -> np.ndarray:
    """E8M0 scales [rows][kblocks] -> the rearranged byte buffer."""
    s = np.asarray(s, np.uint8)
    rows, kb = s.shape
    RT, KT = -(-rows // 32), -(-kb // 8)
    out = np.full((RT, KT, 2, 32, 4), 0x7F, np.uint8)           # [rt][kt][h][r][t]
    padded = np.full((RT * 32, KT * 8), 0x7F, np.uint8)
    padded[:rows, :kb] = s
    # block 8kt + 2t + h of row 32rt + r
    p = padded.reshape(RT, 32, KT, 4, 2)                         # [rt][r][kt][t][h]
    out[:] = p.transpose(0, 2, 4, 1, 3)
    return out.reshape(-1)


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.uint8)
    scale = np.where(s == 255, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127))
    return E4M3[q] * np.repeat(scale, BLOCK, axis=-1)


def gemm(qa, sa, qb, sb):
    """(C, Bnd): deq(A) deq(B)^T and |deq(A)| |deq(B)|^T in float64."""
    da, db = dequantize(qa, sa), dequantize(qb, sb)
    return da @ db.T, np.abs(da) @ np.abs(db).T
