"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test compares the oracle with an independent source: brute-force search
over all 256 E4M3 codes, PyTorch's float8_e4m3fn decoding, a characterisation
of the shared-scale rule, hand-derived golden blocks (tests/golden/), exact
rational arithmetic, closed forms, and the invariants the MXFP8 RL paper relies
on ("End-to-End MXFP8 Reinforcement Learning on Blackwell": power-of-two
scales, Figure 3 / Table 10 row F6; synchronized weights equal byte for byte,
abstract and Table 11 "byte comparison").  All of these run on the CPU.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import mxsynth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# ---------------------------------------------------------------------------
# independent references


def torch_e4m3_table() -> np.ndarray:
    """Values of the 256 E4M3 codes as decoded by PyTorch's float8_e4m3fn dtype."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def bruteforce_encode(t: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code of the same sign as t; ties go to the even code.

    Pure search over the code table: no exponent arithmetic, no rounding
    primitive.  Saturation falls out of it (448 is the nearest finite code to
    anything larger), and so does the signed zero."""
    table = torch_e4m3_table()
    codes = np.arange(256)
    finite = ~np.isnan(table)
    out = np.empty(t.shape, np.uint8)
    neg = np.signbit(t)
    for sign_mask, cand in ((~neg, codes[(codes < 128) & finite]),
                            (neg, codes[(codes >= 128) & finite])):
        idx = np.nonzero(sign_mask)[0]
        vals = table[cand]
        for s in range(0, idx.size, 4096):
            part = idx[s:s + 4096]
            d = np.abs(vals[None, :] - t[part][:, None])
            dmin = d.min(axis=1, keepdims=True)
            tie = d == dmin
            even = tie & (cand[None, :] % 2 == 0)
            pick = np.where(even.any(axis=1, keepdims=True), even, tie)
            out[part] = cand[np.argmax(pick, axis=1)]
    return out


def all_finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def bf16_values(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def exhaustive_t():
    """All (BF16 value, scale code) pairs: t = v / 2^(c-127), exact in float64."""
    v = bf16_values(all_finite_bf16())
    c = np.arange(255)
    t = (v[:, None] * np.ldexp(1.0, 127 - c)[None, :]).ravel()
    return t


# ---------------------------------------------------------------------------
# P1: element encoding


def test_e4m3_decode_matches_torch_float8():
    table = torch_e4m3_table()
    ours = oracle.e4m3_decode_array(np.arange(256, dtype=np.uint8))
    nan = np.isnan(table)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(table[~nan], ours[~nan])
    assert np.array_equal(np.signbit(table[~nan]), np.signbit(ours[~nan]))


def test_e4m3_encode_exhaustive_against_bruteforce():
    """Every BF16 value divided by every power-of-two scale 2^(c-127), c = 0..254
    (16.6 M cases): the oracle's encoder equals nearest-code search.

    Search distances are exact in float64 for 2^-12 <= |t| <= 2^10 (all the
    bits of t - code fit in 53).  Outside that window the nearest code is
    known without search: above 2^10 every finite code lies below t, so the
    largest (448) is nearest; below 2^-12 zero is nearer than 2^-9."""
    t = exhaustive_t()
    ours = oracle.e4m3_encode_array(t)
    a = np.abs(t)
    mid = (a >= 2.0 ** -12) & (a <= 2.0 ** 10)
    # deduplicate by bit pattern so that +0 and -0 stay distinct
    uniq, inv = np.unique(t[mid].view(np.uint64), return_inverse=True)
    ref = bruteforce_encode(uniq.view(np.float64))[inv.ravel()]
    bad = np.nonzero(ours[mid] != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first t={t[mid][bad[0]]!r} " \
                          f"ours={ours[mid][bad[0]]:#x} ref={ref[bad[0]]:#x}"
    sign = np.where(np.signbit(t), 0x80, 0).astype(np.uint8)
    hi = a > 2.0 ** 10
    assert np.array_equal(ours[hi], sign[hi] | 0x7E)
    lo = a < 2.0 ** -12
    assert np.array_equal(ours[lo], sign[lo])
    assert mid.sum() > 1_000_000 and hi.sum() > 0 and lo.sum() > 0


def test_e4m3_encode_matches_torch_conversion_below_overflow():
    """PyTorch's float32 -> float8_e4m3fn conversion rounds to nearest even but
    returns NaN instead of saturating; below 464 the two must agree."""
    v = bf16_values(all_finite_bf16())
    for c in (100, 110, 119, 120, 121, 126, 127, 130, 140):
        t = v * math.ldexp(1.0, 127 - c)
        keep = (np.abs(t) < 464.0) & ((np.abs(t) > 2.0 ** -120) | (t == 0))
        t = t[keep]
        ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3_encode_array(t), ref), c


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode_array(oracle.e4m3_decode_array(codes)), codes)


@pytest.mark.parametrize("mistake", ["half_away", "truncate", "no_subnormals", "nan_on_overflow",
                                     "unsigned_zero"])
def test_bruteforce_pin_catches_planted_encoder_mistakes(mistake):
    """The exhaustive pin has teeth: plausible wrong encoders (written here, in
    numpy, on the CPU) each disagree with the brute-force search somewhere."""
    t = np.unique(exhaustive_t()[::97].view(np.uint64)).view(np.float64)
    t = t[(np.abs(t) <= 1024) & (np.abs(t) >= 2.0 ** -12)]
    a = np.abs(t)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    q = np.ldexp(1.0, (e - 3).astype(int))
    n = a / q
    if mistake == "half_away":
        r = np.floor(n + 0.5) * q
    elif mistake == "truncate":
        r = np.floor(n) * q
    else:
        r = np.rint(n) * q
    if mistake == "no_subnormals":
        r = np.where(r < 2.0 ** -6, 0.0, r)
    r = np.minimum(r, 448.0) if mistake != "nan_on_overflow" else np.where(r > 448, np.nan, r)
    val = np.copysign(r, t) if mistake != "unsigned_zero" else np.where(r == 0, 0.0,
                                                                      np.copysign(r, t))
    table = torch_e4m3_table()
    lut = {(float(table[c]), bool(np.signbit(table[c]))): c for c in range(256)
           if not np.isnan(table[c])}
    wrong = np.array([lut.get((float(x), bool(np.signbit(x))), 0x7F) if not np.isnan(x)
                      else 0x7F for x in val], np.uint8)
    assert (wrong != bruteforce_encode(t)).any()


# ---------------------------------------------------------------------------
# P2: shared-scale rule


def test_scale_rule_characterisation_all_bf16():
    """For every positive finite BF16 amax: scale 2^(c-127) is the power of two
    that puts amax/X in [256, 512) (floor rule with 448 = 1.75 * 2^8), unless
    that would need c < 0, where c clamps to 0."""
    b = all_finite_bf16()
    b = b[(b & 0x8000) == 0]
    amax = bf16_values(b)
    c = oracle.scale_code_array(amax)
    pos = amax > 0
    big = amax >= 2.0 ** -119
    ratio = amax[big] * np.ldexp(1.0, 127 - c[big].astype(int))
    assert ((ratio >= 256) & (ratio < 512)).all()
    assert (c[big] <= 254).all()
    assert (c[pos & ~big] == 0).all()
    assert c[~pos].tolist() == [0]
    assert oracle.scale_code(float("inf")) == 0xFF and oracle.scale_code(float("nan")) == 0xFF


def test_scale_rule_floor_not_ceil():
    """amax = 480 gives X = 1 (480 saturates to 448), not X = 2 (which would keep 240)."""
    assert oracle.scale_code(480.0) == 127
    assert oracle.scale_code(448.0) == 127
    assert oracle.scale_code(511.0) == 127
    assert oracle.scale_code(512.0) == 128
    assert oracle.scale_code(255.99) == 126


# ---------------------------------------------------------------------------
# P3: hand-derived golden blocks


def read_golden_blocks():
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "quantize_blocks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "block":
                cur = {"name": tok[1], "x": [], "val": [], "q": []}
                blocks.append(cur)
            elif tok[0] == "scale":
                cur["s"] = int(tok[1], 16)
            else:
                cur["x"].append(int(tok[0], 16))
                cur["val"].append(float(tok[1]))
                cur["q"].append(int(tok[2], 16))
    return blocks


GOLDEN_BLOCKS = read_golden_blocks()


@pytest.mark.parametrize("blk", GOLDEN_BLOCKS, ids=[b["name"] for b in GOLDEN_BLOCKS])
def test_golden_block(blk):
    assert len(blk["x"]) == 32
    x = np.array(blk["x"], np.uint16)
    # the fixture's printed values and its bit patterns describe the same numbers
    vals = bf16_values(x)
    for v, w in zip(vals, blk["val"]):
        assert (np.isnan(v) and np.isnan(w)) or (v == w and np.signbit(v) == np.signbit(w))
    q, s = oracle.quantize_rowwise(x[None, :])
    assert s[0, 0] == blk["s"]
    assert q[0].tolist() == blk["q"]
    # the same block down a column
    qt, st = oracle.quantize_colwise(x[:, None])
    assert st[0, 0] == blk["s"] and qt[0].tolist() == blk["q"]


# ---------------------------------------------------------------------------
# P4: invariants on config-shaped data


def _sample_tensors():
    A, B = mxsynth.tiny()
    yield "tiny_A", mxsynth.bits(A)
    yield "tiny_B_T", mxsynth.bits(B.t().contiguous())
    yield "weights", mxsynth.bits(mxsynth.normal_bf16((96, 512), 0.02, 7, 0.001, 20.0))
    yield "acts", mxsynth.bits(mxsynth.channel_outliers_bf16(64, 1024, 1.0, 8, 0.005, 50.0))
    yield "grads", mxsynth.bits(mxsynth.normal_bf16((64, 256), 1e-3, 9))


SAMPLES = list(_sample_tensors())


@pytest.mark.parametrize("name,x", SAMPLES, ids=[n for n, _ in SAMPLES])
def test_invariants(name, x):
    q, s = oracle.quantize_rowwise(x)
    # determinism: the same input gives the same bytes (byte-for-byte sync)
    q2, s2 = oracle.quantize_rowwise(x.copy())
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # power-of-two scales only: every scale byte is a finite E8M0 code
    assert (s <= 254).all()
    # no NaN element codes for finite input
    assert not np.isin(q, [0x7F, 0xFF]).any()
    # the block maximum lands in the top E4M3 binade [256, 448] unless the scale clamps
    mags = np.abs(oracle.e4m3_decode_array(q)).reshape(q.shape[0], -1, 32).max(axis=2)
    amax = np.abs(bf16_values(x)).reshape(x.shape[0], -1, 32).max(axis=2)
    E = ((x.astype(np.uint32) & 0x7FFF) >> 7).reshape(x.shape[0], -1, 32).max(axis=2)
    top = E >= 8
    assert ((mags[top] >= 256) & (mags[top] <= 448)).all()
    assert (s[amax == 0] == 0).all()
    # idempotent re-quantization of the dequantized (exactly BF16-representable) values
    deq = oracle.dequantize_rowwise(q, s)
    deq_bits = mxsynth.bits(torch.from_numpy(deq).to(torch.bfloat16))
    assert np.array_equal(bf16_values(deq_bits), deq)
    q3, s3 = oracle.quantize_rowwise(deq_bits)
    assert np.array_equal(q3, q) and np.array_equal(s3, s)
    # sign symmetry: Q(-x) flips only the element sign bits
    qn, sn = oracle.quantize_rowwise(x ^ np.uint16(0x8000))
    assert np.array_equal(sn, s) and np.array_equal(qn, q ^ np.uint8(0x80))
    # power-of-two covariance: Q(2^k x) = (same codes, scale + k) when no clamp binds
    for k in (-9, 5):
        xv = torch.from_numpy(bf16_values(x) * 2.0 ** k).to(torch.bfloat16)
        xk = mxsynth.bits(xv)
        assert np.array_equal(bf16_values(xk), bf16_values(x) * 2.0 ** k)
        qk, sk = oracle.quantize_rowwise(xk)
        nz = s > 0
        assert np.array_equal(sk[nz].astype(int), s[nz].astype(int) + k)
        assert np.array_equal(qk, q)
    # column-wise quantization of X is row-wise quantization of X^T
    qt, st = oracle.quantize_colwise(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q) and np.array_equal(st, s)


def test_tiny_zero_blocks():
    A, B = mxsynth.tiny()
    qa, sa = oracle.quantize_rowwise(mxsynth.bits(A))
    zero = (mxsynth.bits(A).reshape(128, 8, 32) & 0x7FFF).max(axis=2) == 0
    assert zero.sum() == 4
    assert (sa[zero] == 0).all() and (qa.reshape(128, 8, 32)[zero] & 0x7F == 0).all()
    qb, sb = oracle.quantize_colwise(mxsynth.bits(B))
    assert (sb == 0).sum() == 4


# ---------------------------------------------------------------------------
# P5: scale rearrangement


def test_swizzle_golden_positions():
    with open(os.path.join(GOLDEN, "swizzle_positions.txt")) as f:
        lines = [ln.split("#", 1)[0].split() for ln in f]
    lines = [ln for ln in lines if ln]
    assert lines[0][0] == "size"
    rows, kb, size = map(int, lines[0][1:])
    assert oracle.swizzled_bytes(rows, kb) == size
    s = np.arange(rows * kb, dtype=np.int64).reshape(rows, kb)
    s8 = (s % 251).astype(np.uint8)  # distinct-enough payload, never 0x7F... checked below
    buf = oracle.scale_swizzle(s8)
    for r, b, off in (map(int, ln) for ln in lines[1:]):
        assert oracle.swizzle_offset(r, b, kb) == off
        assert buf[off] == s8[r, b]


@pytest.mark.parametrize("rows,kb", [(1, 1), (32, 8), (33, 9), (128, 8), (100, 24), (64, 768)])
def test_swizzle_bijective_and_padded(rows, kb):
    n = oracle.swizzled_bytes(rows, kb)
    offs = np.array([[oracle.swizzle_offset(r, b, kb) for b in range(kb)] for r in range(rows)])
    assert offs.min() >= 0 and offs.max() < n
    assert np.unique(offs).size == rows * kb
    rng = np.random.default_rng(rows * 1000 + kb)
    s = rng.integers(0, 255, size=(rows, kb), dtype=np.uint8)
    buf = oracle.scale_swizzle(s)
    pad = np.ones(n, bool)
    pad[offs.ravel()] = False
    assert (buf[pad] == 0x7F).all()
    assert np.array_equal(oracle.scale_unswizzle(buf, rows, kb), s)


# ---------------------------------------------------------------------------
# P6: GEMM


def _random_codes(rng, shape):
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38
    return q


def test_gemm_exact_rational_tiny():
    """Against exact rational arithmetic (fractions.Fraction) on decoded codes:
    the double-precision sum is within K * 2^-53 * Bnd of the exact value."""
    rng = np.random.default_rng(1)
    M, N, K = 3, 4, 96
    qa, qb = _random_codes(rng, (M, K)), _random_codes(rng, (N, K))
    sa = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    table = torch_e4m3_table()
    C, Bnd = oracle.gemm(qa, sa, qb, sb)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(table[qa[i, k]])) * Fraction(2) ** (int(sa[i, k // 32]) - 127)
                        * Fraction(float(table[qb[j, k]])) * Fraction(2) ** (int(sb[j, k // 32]) - 127)
                        for k in range(K))
            bound = sum(abs(Fraction(float(table[qa[i, k]]))) * Fraction(2) ** (int(sa[i, k // 32]) - 127)
                        * abs(Fraction(float(table[qb[j, k]]))) * Fraction(2) ** (int(sb[j, k // 32]) - 127)
                        for k in range(K))
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(K) * Fraction(2) ** -53 * bound
            assert Fraction(Bnd[i, j]) == bound or abs(Fraction(Bnd[i, j]) - bound) <= \
                Fraction(K) * Fraction(2) ** -53 * bound


def test_gemm_closed_forms():
    K = 256
    # all elements 1.0 (0x38) with scale codes cA, cB: C = K * 2^(cA + cB - 254)
    qa = np.full((4, K), 0x38, np.uint8)
    qb = np.full((5, K), 0x38, np.uint8)
    sa = np.full((4, K // 32), 120, np.uint8)
    sb = np.full((5, K // 32), 131, np.uint8)
    C, Bnd = oracle.gemm(qa, sa, qb, sb)
    assert (C == K * 2.0 ** (120 + 131 - 254)).all() and (Bnd == C).all()
    # one-hot A rows select dequantized B entries exactly
    rng = np.random.default_rng(3)
    qb = _random_codes(rng, (6, K))
    sb = rng.integers(100, 150, size=(6, K // 32)).astype(np.uint8)
    qa = np.zeros((3, K), np.uint8)
    sa = np.full((3, K // 32), 127, np.uint8)
    picks = [5, 64, 255]
    for i, k in enumerate(picks):
        qa[i, k] = 0x38
    C, _ = oracle.gemm(qa, sa, qb, sb)
    table = torch_e4m3_table()
    for i, k in enumerate(picks):
        for j in range(6):
            assert C[i, j] == table[qb[j, k]] * 2.0 ** (int(sb[j, k // 32]) - 127)
    # negating A negates C exactly
    qa = _random_codes(rng, (3, K))
    sa = rng.integers(110, 140, size=(3, K // 32)).astype(np.uint8)
    C1, _ = oracle.gemm(qa, sa, qb, sb)
    C2, _ = oracle.gemm(qa ^ np.uint8(0x80), sa, qb, sb)
    assert np.array_equal(C1, -C2)


def test_gemm_sampled_and_grouped_consistent():
    rng = np.random.default_rng(4)
    K, N = 128, 8
    qa = _random_codes(rng, (20, K))
    sa = rng.integers(115, 135, size=(20, K // 32)).astype(np.uint8)
    qb = _random_codes(rng, (3, N, K))
    sb = rng.integers(115, 135, size=(3, N, K // 32)).astype(np.uint8)
    offsets = np.array([0, 7, 7, 20])  # an empty expert in the middle
    Cg, Bg = oracle.grouped_gemm(offsets, qa, sa, qb, sb)
    for g in range(3):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            Cd, Bd = oracle.gemm(qa[lo:hi], sa[lo:hi], qb[g], sb[g])
            assert np.array_equal(Cg[lo:hi], Cd) and np.array_equal(Bg[lo:hi], Bd)
    rows = np.array([0, 19, 6, 7])
    cols = np.array([1, 7, 0, 3])
    Cs, _ = oracle.grouped_gemm_sampled(rows, cols, offsets, qa, sa, qb, sb)
    assert np.array_equal(Cs, Cg[rows, cols])
    # against numpy's float64 matmul of the dequantized operands (a textbook routine)
    Ad = oracle.dequantize_rowwise(qa, sa)
    Bd = oracle.dequantize_rowwise(qb[2], sb[2])
    ref = Ad[7:20] @ Bd.T
    assert (np.abs(Cg[7:20] - ref) <= 1e-12 * (np.abs(Ad[7:20]) @ np.abs(Bd).T)).all()
