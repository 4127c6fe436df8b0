"""The two CPU oracles against each other.

oracle/mx_oracle.c rounds to E4M3 by exponent and mantissa arithmetic and
takes floor(log2 amax) from the BF16 exponent; oracle/mx_oracle_ref.py finds
the nearest value by a search over the table of all finite E4M3 values and
takes the exponent from numpy's frexp.  They must give the same bytes on the
Tiny workload and on 10^6 random 32-element blocks that cover every BF16
exponent, subnormal inputs, zero blocks, ties, saturating blocks and NaN/Inf
blocks; the same rearranged scale bytes; and GEMM results within 1e-12 of
(|A||B|)_ij of each other and of numpy's float64 matrix product.
"""
import numpy as np
import torch

import mxsynth
import oracle
from oracle import mx_oracle_ref as ref


def _random_blocks(n_blocks: int, seed: int) -> np.ndarray:
    """BF16 bit patterns [n_blocks/32][1024] (32 blocks per row)."""
    rng = np.random.default_rng(seed)
    n = n_blocks * 32
    kind = rng.integers(0, 6, size=n_blocks)
    bits = np.empty((n_blocks, 32), np.uint16)
    # 0: uniform random bit patterns (every exponent), NaN/Inf patterns replaced
    u = rng.integers(0, 1 << 16, size=(n_blocks, 32), dtype=np.uint32).astype(np.uint16)
    u[(u & 0x7F80) == 0x7F80] &= 0xBF7F
    # 1: normal data at a random per-block magnitude 2^[-135, 125]
    g = rng.standard_normal((n_blocks, 32)).astype(np.float32)
    g *= np.ldexp(np.float32(1.0), rng.integers(-135, 126, size=(n_blocks, 1))).astype(np.float32)
    gb = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # 2: exact ties and near-ties of the E4M3 grid after scaling: values
    #    (k + 0.5) * 2^-3 * 2^e around a block maximum of 2^(e+8)
    e = rng.integers(-100, 100, size=(n_blocks, 1))
    kk = rng.integers(8, 16, size=(n_blocks, 32)) + rng.choice([0.5, 0.5, 0.25, 0.75], size=(n_blocks, 32))
    sgn = rng.choice([-1.0, 1.0], size=(n_blocks, 32))
    t = (sgn * kk * np.ldexp(1.0, rng.integers(-9, 6, size=(n_blocks, 32)))).astype(np.float64)
    t[:, 0] = 448.0 + rng.choice([0.0, 8.0, 16.0, 24.0, 40.0, 63.0], size=n_blocks)   # saturation region
    tb = torch.from_numpy((t * np.ldexp(1.0, e)).astype(np.float32)).to(torch.bfloat16)
    tb = tb.view(torch.int16).numpy().view(np.uint16)
    # 3: subnormal BF16 inputs and tiny amax
    sub = rng.integers(0, 0x80, size=(n_blocks, 32)).astype(np.uint16) | (rng.integers(0, 2, size=(n_blocks, 32)).astype(np.uint16) << 15)
    # 4: zero blocks (signed zeros), one outlier among them now and then
    z = np.where(rng.random((n_blocks, 32)) < 0.5, 0x8000, 0x0000).astype(np.uint16)
    z[rng.random(n_blocks) < 0.3, 7] = 0x3F80
    # 5: blocks holding NaN or Inf
    s5 = u.copy()
    s5[np.arange(n_blocks), rng.integers(0, 32, size=n_blocks)] = rng.choice(
        np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16), size=n_blocks)
    for k, src in enumerate((u, gb, tb, sub, z, s5)):
        bits[kind == k] = src[kind == k]
    return bits.reshape(n_blocks // 32, 1024)


def test_tiny_bytes_and_gemm_agree():
    A, B = mxsynth.tiny()
    ab, bb = mxsynth.bits(A), mxsynth.bits(B)
    qa, sa = oracle.quantize_rowwise(ab)
    qa2, sa2 = ref.quantize_rowwise(ab)
    assert np.array_equal(qa, qa2) and np.array_equal(sa, sa2)
    qb, sb = oracle.quantize_colwise(bb)
    qb2, sb2 = ref.quantize_colwise(bb)
    assert np.array_equal(qb, qb2) and np.array_equal(sb, sb2)
    for s in (sa, sb):
        assert np.array_equal(oracle.scale_swizzle(s), ref.scale_swizzle(s))
    C, bnd = oracle.gemm(qa, sa, qb, sb)
    C2, bnd2 = ref.gemm(qa, sa, qb, sb)
    assert np.all(np.abs(C - C2) <= 1e-12 * bnd)
    assert np.allclose(bnd, bnd2, rtol=1e-12, atol=0)
    da, db = oracle.dequantize_rowwise(qa, sa), oracle.dequantize_rowwise(qb, sb)
    assert np.array_equal(da, ref.dequantize(qa, sa))
    assert np.all(np.abs(C - np.matmul(da, db.T)) <= 1e-12 * bnd)


def test_million_random_blocks_agree():
    bits = _random_blocks(1 << 20, seed=8)          # 1 048 576 blocks of 32
    q1, s1 = oracle.quantize_rowwise(bits)
    q2, s2 = ref.quantize_rowwise(bits)
    bad = np.argwhere(q1 != q2)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {tuple(bad[0])}: {q1[tuple(bad[0])]:#x} vs {q2[tuple(bad[0])]:#x}"
    assert np.array_equal(s1, s2)
    # the draw reaches every scale code the BF16 range allows, and the specials
    assert set(np.unique(s1).tolist()) >= set(range(0, 247)) | {255}
    assert (q1 == 0x7E).any() and (q1 == 0x80).any() and (q1 == 0x01).any()


def test_colwise_and_rearrangement_agree_on_random_blocks():
    bits = _random_blocks(1 << 15, seed=9).reshape(-1, 256)       # 4096 x 256
    q1, s1 = oracle.quantize_colwise(bits)
    q2, s2 = ref.quantize_colwise(bits)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    for rows, kb in ((256, 128), (200, 100), (33, 9), (1, 1)):
        s = s1[:rows, :kb]
        assert np.array_equal(oracle.scale_swizzle(np.ascontiguousarray(s)), ref.scale_swizzle(s))
