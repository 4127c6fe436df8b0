"""Pins of the oracle's MoE backward pieces (CPU).

The expert weight gradient dW_g = dY_g^T X_g ("End-to-End MXFP8 Reinforcement
Learning on Blackwell", Table 8: update_actor of the MoE learner; Table 2:
128 experts, top-8) contracts over the expert's own token rows, with both
operands quantized column-wise in 32-row blocks that stay inside one expert.

Pins, each chosen so a plausible mistake fails one of them:
  - the padded column ranges, against values derived by hand;
  - the grouped column-wise quantizer, against a loop over single elements
    built from the scalar encoder and scale rule (themselves pinned by brute
    force), and against a planted straddling block;
  - the per-expert product, against exact rational arithmetic on a tiny case,
    numpy float64 products of the dequantized slices, and the unquantized
    product dY_g^T X_g within the E4M3 rounding bound (which catches a swapped
    or transposed operand)."""
from fractions import Fraction

import numpy as np
import torch

import mxsynth
import oracle


def test_pad_offsets_hand_values():
    # m = 0, 1, 255, 256, 257, 600 -> 256, 256, 256, 256, 512, 768
    pad = oracle.grouped_pad_offsets([0, 0, 1, 256, 512, 769, 1369])
    assert pad.tolist() == [0, 256, 512, 768, 1024, 1536, 2304]
    assert oracle.grouped_pad_offsets([0, 1024]).tolist() == [0, 1024]
    assert oracle.grouped_pad_offsets([0, 1025]).tolist() == [0, 1280]
    # the capacity bound holds for every split
    rng = np.random.default_rng(0)
    for _ in range(50):
        G = int(rng.integers(1, 20))
        cut = np.sort(rng.integers(0, 3000, size=G - 1))
        off = np.concatenate([[0], cut, [3000]])
        assert oracle.grouped_pad_offsets(off)[-1] <= oracle.grouped_k_capacity(3000, G)


def _loop_colwise_grouped(xb, off, pad, k_cap):
    """Column-wise blocks of each expert's rows, one element at a time."""
    rows, cols = xb.shape
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qt = np.zeros((cols, k_cap), np.uint8)
    st = np.zeros((cols, k_cap // 32), np.uint8)
    for g in range(len(off) - 1):
        for c in range(cols):
            for b in range((pad[g + 1] - pad[g]) // 32):
                vals = [x[r, c] if r < off[g + 1] else 0.0
                        for r in range(off[g] + 32 * b, off[g] + 32 * b + 32)]
                code = oracle.scale_code(max(abs(v) for v in vals))
                st[c, pad[g] // 32 + b] = code
                X = 2.0 ** (code - 127)
                for i, v in enumerate(vals):
                    qt[c, pad[g] + 32 * b + i] = oracle.e4m3_encode(v / X)
    return qt, st


def test_colwise_grouped_equals_element_loop():
    sizes = [0, 37, 256, 300, 5]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rows, cols = int(off[-1]), 8
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=11, outlier_frac=0.02)
    xb = mxsynth.bits(x)
    k_cap = oracle.grouped_k_capacity(rows, len(sizes))
    qt, st, pad = oracle.quantize_colwise_grouped(xb, off, k_cap)
    eqt, est = _loop_colwise_grouped(xb, off, oracle.grouped_pad_offsets(off), k_cap)
    assert np.array_equal(qt, eqt) and np.array_equal(st, est)
    # the empty expert's range is all zero codes with scale 0
    assert (qt[:, pad[0]:pad[1]] == 0).all() and (st[:, pad[0] // 32:pad[1] // 32] == 0).all()
    # rows past an expert's count are zero codes
    assert (qt[:, pad[1] + 37:pad[2]] == 0).all()


def test_colwise_grouped_block_does_not_straddle_experts():
    # expert 0 has 40 rows of 1.0; expert 1's first row is 2^20.  A block that
    # straddled the boundary (rows 32..63 of the whole tensor) would take its
    # scale from 2^20 and flush expert 0's ones to zero.
    rows, cols = 80, 8
    x = torch.ones(rows, cols, dtype=torch.float32)
    x[40] = 2.0 ** 20
    xb = mxsynth.bits(x.to(torch.bfloat16))
    off = np.array([0, 40, 80], np.int64)
    qt, st, pad = oracle.quantize_colwise_grouped(xb, off, 1024)
    assert pad.tolist() == [0, 256, 512]
    # expert 0, block 1 (its rows 32..39 plus zeros): amax 1 -> code 127 - 8 = 119
    assert (st[:, 1] == 119).all()
    assert (qt[:, 32:40] == 0x78).all()   # 1.0 / 2^-8 = 256 = 2^8 -> E4M3 0x78 (e = 8 + 7, m = 0)
    assert (qt[:, 40:64] == 0).all()
    # expert 1, block 0: amax 2^20 -> code 127 + 12 = 139; its other rows (1.0)
    # are 2^-12 of the scale, below E4M3's smallest subnormal 2^-9: zero
    assert (st[:, pad[1] // 32] == 139).all()
    assert (qt[:, pad[1]] == 0x78).all() and (qt[:, pad[1] + 1:pad[1] + 32] == 0).all()


def _random_codes(rng, shape):
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C   # no NaN codes
    return q


def test_wgrad_exact_rational_tiny():
    rng = np.random.default_rng(7)
    pad = np.array([0, 64, 64 + 96, 64 + 96 + 32], np.int64)
    Kc = 256
    M, N = 3, 2
    qa, qb = _random_codes(rng, (M, Kc)), _random_codes(rng, (N, Kc))
    sa = rng.integers(120, 135, size=(M, Kc // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, size=(N, Kc // 32)).astype(np.uint8)

    def deq(q, s):
        v = Fraction(oracle.e4m3_decode(int(q)))
        return v * Fraction(2) ** (int(s) - 127)

    c, bnd = oracle.grouped_wgrad(pad, qa, sa, qb, sb)
    for g in range(3):
        for i in range(M):
            for j in range(N):
                ex = sum(deq(qa[i, k], sa[i, k // 32]) * deq(qb[j, k], sb[j, k // 32])
                         for k in range(pad[g], pad[g + 1]))
                eb = sum(abs(deq(qa[i, k], sa[i, k // 32]) * deq(qb[j, k], sb[j, k // 32]))
                         for k in range(pad[g], pad[g + 1]))
                assert abs(Fraction(c[g, i, j]) - ex) <= Fraction(1, 2 ** 40) * eb
                assert abs(Fraction(bnd[g, i, j]) - eb) <= Fraction(1, 2 ** 40) * eb


def test_wgrad_slices_match_numpy_and_add_up():
    rng = np.random.default_rng(8)
    pad = np.array([0, 256, 768, 1024], np.int64)
    Kc, M, N = 1280, 40, 24
    qa, qb = _random_codes(rng, (M, Kc)), _random_codes(rng, (N, Kc))
    sa = rng.integers(118, 136, size=(M, Kc // 32)).astype(np.uint8)
    sb = rng.integers(118, 136, size=(N, Kc // 32)).astype(np.uint8)
    da, db = oracle.dequantize_rowwise(qa, sa), oracle.dequantize_rowwise(qb, sb)
    c, bnd = oracle.grouped_wgrad(pad, qa, sa, qb, sb)
    total = np.zeros((M, N))
    for g in range(3):
        ref = da[:, pad[g]:pad[g + 1]] @ db[:, pad[g]:pad[g + 1]].T
        tol = 1e-12 * (np.abs(da[:, pad[g]:pad[g + 1]]) @ np.abs(db[:, pad[g]:pad[g + 1]]).T)
        assert (np.abs(c[g] - ref) <= tol).all()
        total += c[g]
    # columns past pad[G] take no part: the ranges add up to the product over [0, pad[G])
    full = da[:, :pad[-1]] @ db[:, :pad[-1]].T
    assert np.allclose(total, full, rtol=0, atol=1e-10 * np.abs(full).max())


def test_wgrad_matches_unquantized_gradient():
    """dW_g = dY_g^T X_g from the BF16 inputs, within E4M3's rounding bound."""
    sizes = [70, 0, 200, 33]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    T, Nout, Kin = int(off[-1]), 64, 32
    dy = mxsynth.normal_bf16((T, Nout), 1e-3, seed=21)
    x = mxsynth.normal_bf16((T, Kin), 1.0, seed=22)
    k_cap = oracle.grouped_k_capacity(T, len(sizes))
    qa, sa, pad = oracle.quantize_colwise_grouped(mxsynth.bits(dy), off, k_cap)
    qb, sb, _ = oracle.quantize_colwise_grouped(mxsynth.bits(x), off, k_cap)
    c, bnd = oracle.grouped_wgrad(pad, qa, sa, qb, sb)
    assert c.shape == (len(sizes), Nout, Kin)
    dyf = dy.double().numpy()
    xf = x.double().numpy()
    for g in range(len(sizes)):
        ref = dyf[off[g]:off[g + 1]].T @ xf[off[g]:off[g + 1]]
        absb = np.abs(dyf[off[g]:off[g + 1]]).T @ np.abs(xf[off[g]:off[g + 1]])
        # |deq(a) - a| <= 2^-4 |a| for E4M3 normals (3 mantissa bits, nearest);
        # subnormal codes add at most 2^-10 of the block scale each
        assert (np.abs(c[g] - ref) <= 0.13 * absb + 1e-9).all()
        if sizes[g] == 0:
            assert (c[g] == 0).all()
