"""GPU parity of the dense and grouped block-scaled GEMMs.

Bar: |C - C_model| <= 1e-5 * (|A||B|)_ij elementwise, plus one BF16 ulp for
BF16 output, where C_model is the exact sum of the products as the matrix
cores' 8-product window truncates them (tests/mfma_model.py, pinned bit for
bit on the GPU by tests/test_gpu_mfma_model.py); C exactly zero where every
product is zero.  (|A||B|)_ij and the exact result come from the oracle; how
many outputs also meet the stated bar against the exact result is reported.
Cases whose every product is exact in that window (single nonzeros, equal
values) are checked for exact equality.
"""
import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import (assert_gemm_close, bf16_dev, full_range_codes, gemm_ref, grouped_ref,
                      random_mx_operand, to_dev)

pytestmark = pytest.mark.gpu


def _run(mx, qa, sa, qb, sb, out_dtype):
    a_swz = mx.mx_scale_swizzle(to_dev(sa))
    b_swz = mx.mx_scale_swizzle(to_dev(sb))
    return mx.mx_gemm(to_dev(qa), a_swz, to_dev(qb), b_swz, out_dtype=out_dtype)


def test_tiny_config_end_to_end(gpu_lib):
    """A[128x256] row-wise, B[256x256] column-wise, swizzle, 128x256x256 GEMM."""
    mx = gpu_lib
    A, B = mxsynth.tiny()
    qa, sa = mx.mx_quantize_rowwise(bf16_dev(A))
    qbt, sbt = mx.mx_quantize_colwise(bf16_dev(B))
    a_swz, b_swz = mx.mx_scale_swizzle(sa), mx.mx_scale_swizzle(sbt)
    oqa, osa = oracle.quantize_rowwise(mxsynth.bits(A))
    oqb, osb = oracle.quantize_colwise(mxsynth.bits(B))
    r = gemm_ref(oqa, osa, oqb, osb)
    from gpu_util import stats_line
    for dt in (torch.bfloat16, torch.float32):
        C = mx.mx_gemm(qa, a_swz, qbt, b_swz, out_dtype=dt)
        print(stats_line(f"tiny 128x256x256 {dt}", assert_gemm_close(C, r, f"tiny {dt}")))


@pytest.mark.parametrize("M,N,K", [(32, 32, 128), (256, 256, 256), (300, 520, 384),
                                   (1, 7, 128), (513, 260, 1152), (64, 1000, 2048)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_random_shapes(gpu_lib, M, N, K, out_dtype):
    """Several tiles, ragged M and N tails, K with a half 256-K scale group."""
    mx = gpu_lib
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    qa, sa = random_mx_operand(rng, M, K)
    qb, sb = random_mx_operand(rng, N, K)
    r = gemm_ref(qa, sa, qb, sb)
    C = _run(mx, qa, sa, qb, sb, out_dtype)
    assert_gemm_close(C, r, f"{M}x{N}x{K}")


def test_strided_output_and_operands(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(5)
    M, N, K = 200, 136, 256
    qa, sa = random_mx_operand(rng, M, K + 64)
    qb, sb = random_mx_operand(rng, N, K + 128)
    a_dev = to_dev(qa)[:, :K]          # ld_a = K + 64
    b_dev = to_dev(qb)[:, :K]          # ld_b = K + 128
    r = gemm_ref(qa[:, :K].copy(), sa[:, :K // 32].copy(), qb[:, :K].copy(),
                 sb[:, :K // 32].copy())
    cbuf = torch.full((M, N + 12), 7.0, dtype=torch.float32, device="cuda")
    C = mx.mx_gemm(a_dev, mx.mx_scale_swizzle(to_dev(sa)[:, :K // 32]), b_dev,
                   mx.mx_scale_swizzle(to_dev(sb)[:, :K // 32]), c=cbuf[:, :N])
    assert_gemm_close(C, r, "strided")
    assert (cbuf[:, N:] == 7.0).all()


def test_single_nonzero_probes(gpu_lib):
    """One nonzero code per operand: maps lane, row, K-block and scale byte
    placement.  Each output is a single exact product, so any misplacement
    shows as a wrong position or a wrong power of two."""
    mx = gpu_lib
    M, N, K = 64, 64, 512
    rng = np.random.default_rng(17)
    for trial in range(12):
        i, j, k = int(rng.integers(M)), int(rng.integers(N)), int(rng.integers(K))
        qa = np.zeros((M, K), np.uint8)
        qb = np.zeros((N, K), np.uint8)
        qa[i, k] = 0x38 + int(rng.integers(0, 7))           # 1.0 .. 1.75
        qb[j, k] = 0x40 + int(rng.integers(0, 7))           # 2.0 .. 3.5
        sa = rng.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
        ref, bnd = oracle.gemm(qa, sa, qb, sb)
        C = _run(mx, qa, sa, qb, sb, torch.float32).cpu().numpy()
        expect = np.zeros((M, N))
        expect[i, j] = ref[i, j]
        assert ref[i, j] != 0
        assert np.array_equal(C, expect), f"trial {trial}: (i,j,k)=({i},{j},{k})"


def test_closed_forms(gpu_lib):
    mx = gpu_lib
    M, N, K = 96, 80, 1024
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((N, K), 0x38, np.uint8)
    sa = np.full((M, K // 32), 120, np.uint8)
    sb = np.full((N, K // 32), 131, np.uint8)
    C = _run(mx, qa, sa, qb, sb, torch.float32).cpu().numpy()
    assert (C == K * 2.0 ** (120 + 131 - 254)).all()
    # negating A negates C within the bar.  Bit for bit only per run of 8: the
    # truncation inside a run is toward zero (sign-symmetric, pinned bitwise in
    # tests/test_gpu_mfma_model.py), but the FP32 addition of run sums rounds
    # a smaller addend down (toward -inf) at about 2^-24 of the larger, so a
    # general negated product may differ in its last bits.
    rng = np.random.default_rng(8)
    qa, sa = random_mx_operand(rng, M, K)
    qb, sb = random_mx_operand(rng, N, K)
    r = gemm_ref(qa, sa, qb, sb)
    C1 = _run(mx, qa, sa, qb, sb, torch.float32)
    C2 = _run(mx, qa ^ np.uint8(0x80), sa, qb, sb, torch.float32)
    assert_gemm_close(C1, r, "A")
    assert_gemm_close(-C2, r, "-(-A)")


def test_stale_swizzled_scales_detected(gpu_lib):
    """New weights with the old rearranged scales (paper Table 10, F3; Table 13
    'new weights with stale derived scales') must fail the parity check."""
    mx = gpu_lib
    A, B = mxsynth.tiny()
    B2 = (B.float() * 4.0 + 0.5).to(torch.bfloat16)
    qa, sa = mx.mx_quantize_rowwise(bf16_dev(A))
    qbt, sbt = mx.mx_quantize_colwise(bf16_dev(B))
    stale = mx.mx_scale_swizzle(sbt)
    qbt2, sbt2 = mx.mx_quantize_colwise(bf16_dev(B2))
    oqa, osa = oracle.quantize_rowwise(mxsynth.bits(A))
    oqb2, osb2 = oracle.quantize_colwise(mxsynth.bits(B2))
    r = gemm_ref(oqa, osa, oqb2, osb2)
    C_stale = mx.mx_gemm(qa, mx.mx_scale_swizzle(sa), qbt2, stale, out_dtype=torch.float32)
    with pytest.raises(AssertionError):
        assert_gemm_close(C_stale, r, "stale")
    C_fresh = mx.mx_gemm(qa, mx.mx_scale_swizzle(sa), qbt2, mx.mx_scale_swizzle(sbt2),
                         out_dtype=torch.float32)
    assert_gemm_close(C_fresh, r, "fresh")


@pytest.mark.parametrize("M,N,K", [(700, 768, 512), (512, 512, 2048), (300, 256, 1280),
                                   (256, 512, 1152), (33, 256, 4096)])
def test_split_tail_matches_oracle(gpu_lib, M, N, K):
    """Tile counts that leave a partial round of workgroups: the leftover
    tiles are cut into K ranges of whole 256-K groups (2 to 8 ranges here,
    one group per range for K = 1280, the padded half group for K = 1152)
    whose FP32 partial tiles are summed by the last range to finish."""
    mx = gpu_lib
    rng = np.random.default_rng(M + N + K)
    qa, sa = random_mx_operand(rng, M, K)
    qb, sb = random_mx_operand(rng, N, K)
    C = _run(mx, qa, sa, qb, sb, torch.bfloat16)
    assert_gemm_close(C, gemm_ref(qa, sa, qb, sb), f"split tail {M}x{N}x{K}")
    assert torch.equal(C, _run(mx, qa, sa, qb, sb, torch.bfloat16))


def test_split_tail_after_full_rounds(gpu_lib):
    """272 tiles on 256 compute units: one whole tile per workgroup, then the
    last 16 tiles split in two K ranges; sampled outputs, the split rows
    (the last 256-row band) sampled densely."""
    from gpu_util import check_sampled, sample_entries
    mx = gpu_lib
    M, N, K = 4352, 4096, 512
    rng = np.random.default_rng(272)
    qa, sa = random_mx_operand(rng, M, K)
    qb, sb = random_mx_operand(rng, N, K)
    C = _run(mx, qa, sa, qb, sb, torch.bfloat16)
    rows, cols = sample_entries(rng, M, N)
    rows = np.concatenate([rows, rng.integers(M - 256, M, size=2048)])
    cols = np.concatenate([cols, rng.integers(0, N, size=2048)])
    check_sampled(C, rows, cols, qa, sa, qb, sb, "split tail after a full round")
    assert torch.equal(C, _run(mx, qa, sa, qb, sb, torch.bfloat16))


def test_gemm_deterministic(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(21)
    qa, sa = random_mx_operand(rng, 512, 2048)
    qb, sb = random_mx_operand(rng, 512, 2048)
    C1 = _run(mx, qa, sa, qb, sb, torch.bfloat16)
    C2 = _run(mx, qa, sa, qb, sb, torch.bfloat16)
    assert torch.equal(C1, C2)


# ---------------------------------------------------------------------------
# grouped (per-expert) GEMM


def _grouped_case(rng, sizes, N, K):
    sizes = np.asarray(sizes, np.int64)
    M = int(sizes.sum())
    G = sizes.size
    qa, sa = random_mx_operand(rng, M, K)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N, K // 32), np.uint8)
    for g in range(G):
        qb[g], sb[g] = random_mx_operand(rng, N, K)
    return mxsynth.offsets_from_rows(sizes), qa, sa, qb, sb


def _run_grouped(mx, off, qa, sa, qb, sb, out_dtype):
    G, N, K = qb.shape
    a_swz = mx.mx_scale_swizzle(to_dev(sa))
    b_swz = torch.cat([mx.mx_scale_swizzle(to_dev(sb[g])) for g in range(G)])
    return mx.mx_grouped_gemm(to_dev(off), to_dev(qa), a_swz, to_dev(qb), b_swz,
                              out_dtype=out_dtype)


@pytest.mark.parametrize("sizes,N,K", [([300], 256, 256), ([5, 0, 260, 33, 0, 512, 1], 192, 384),
                                       ([0, 0, 70], 64, 128), ([256, 256], 300, 512),
                                       ([17] * 9, 520, 256)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_matches_oracle(gpu_lib, sizes, N, K, out_dtype):
    mx = gpu_lib
    rng = np.random.default_rng(sum(sizes) * 13 + N + K)
    off, qa, sa, qb, sb = _grouped_case(rng, sizes, N, K)
    r = grouped_ref(off, qa, sa, qb, sb)
    C = _run_grouped(mx, off, qa, sa, qb, sb, out_dtype)
    assert_gemm_close(C, r, f"grouped {sizes}")


def test_grouped_single_group_equals_dense(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(3)
    off, qa, sa, qb, sb = _grouped_case(rng, [700], 384, 512)
    Cg = _run_grouped(mx, off, qa, sa, qb, sb, torch.float32)
    Cd = _run(mx, qa, sa, qb[0], sb[0], torch.float32)
    assert torch.equal(Cg, Cd)


def test_grouped_permuted_experts_detected(gpu_lib):
    """Same shape and dtype, experts swapped (paper Table 10, F4; Table 13
    'content permuted, shape and dtype kept'): the check must fail."""
    mx = gpu_lib
    rng = np.random.default_rng(4)
    off, qa, sa, qb, sb = _grouped_case(rng, [64, 100, 90], 128, 256)
    r = grouped_ref(off, qa, sa, qb, sb)
    perm = [1, 0, 2]
    C = _run_grouped(mx, off, qa, sa, qb[perm].copy(), sb[perm].copy(), torch.float32)
    with pytest.raises(AssertionError):
        assert_gemm_close(C, r, "permuted")


def test_grouped_last_expert_corruption_detected(gpu_lib):
    """Corruption confined to the last expert (paper Table 13: a probe of the
    first expert is blind to it) is caught because every expert is checked."""
    mx = gpu_lib
    rng = np.random.default_rng(6)
    off, qa, sa, qb, sb = _grouped_case(rng, [40, 50, 60, 70], 96, 256)
    r = grouped_ref(off, qa, sa, qb, sb)
    qb_bad = qb.copy()
    k = int(np.nonzero(qb[-1, 5] & 0x7F)[0][0])   # a nonzero code: flipping its sign matters
    qb_bad[-1, 5, k] ^= 0x80
    C = _run_grouped(mx, off, qa, sa, qb_bad, sb, torch.float32)
    first = slice(0, int(off[1]))
    assert_gemm_close(C[first], r[first], "first expert only")
    with pytest.raises(AssertionError):
        assert_gemm_close(C, r, "all experts")


def test_full_range_codes_against_model(gpu_lib):
    """Uniformly random E4M3 codes (every exponent, subnormals included) span
    far more than 13 binades inside a run of 8, so the window truncation is
    exercised hard: the GEMM stays within the stated bar of the model, and
    the stated bar against the exact sum fails somewhere (the model is
    needed, not slack)."""
    mx = gpu_lib
    rng = np.random.default_rng(99)
    M, N, K = 96, 160, 512
    qa, sa = full_range_codes(rng, M, K)
    qb, sb = full_range_codes(rng, N, K)
    r = gemm_ref(qa, sa, qb, sb)
    C = _run(mx, qa, sa, qb, sb, torch.float32)
    stats = assert_gemm_close(C, r, "full range")
    assert stats["within_stated"] < stats["n"]
