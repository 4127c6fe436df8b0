"""GPU parity of the MoE backward products against the oracle.

The expert weight gradient dW_g = dY_g^T X_g ("End-to-End MXFP8 Reinforcement
Learning on Blackwell", Table 8: update_actor; Table 2: Qwen3-30B-A3B, 128
experts, top-8) runs as mx_quantize_colwise_grouped of dY and X (per-expert
column-wise blocks in 256-aligned column ranges) followed by
mx_grouped_gemm_wgrad; the data gradient dX = dY . W_g per expert is
mx_grouped_gemm with the column-wise expert weights of
mx_quantize_dual_experts.  Quantized bytes are compared bit for bit; GEMM
outputs at the stated bar against the run-window model of tests/gpu_util.py
(1e-5 * (|A||B|)_ij, plus one BF16 ulp for BF16 output), with the count
that also meets it against the oracle's exact result reported.  Full-size
products are checked on lattices reaching every 256 x 256 tile of every
expert.
"""
import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import (_pool_map, assert_gemm_close, check_sampled_grouped, check_sampled_wgrad,
                      lattice_grouped, lattice_wgrad, oracle_colwise_par, stats_line, wgrad_ref)

pytestmark = pytest.mark.gpu


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def _grouped_oracle_par(xb, off, k_cap, chunk=256):
    """oracle.quantize_colwise_grouped split over column chunks (threads)."""
    cols = xb.shape[1]
    parts = _pool_map(lambda c0: oracle.quantize_colwise_grouped(
        np.ascontiguousarray(xb[:, c0:c0 + chunk]), off, k_cap), range(0, cols, chunk))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            parts[0][2])


def _check_grouped_quant(mx, x, off, what, sentinel=True):
    """Run the grouped quantizer on x (CPU BF16) and compare with the oracle:
    pad offsets, codes up to pad[G], rearranged scale tiles up to pad[G], and
    (sentinel) nothing written past pad[G].  Returns GPU and oracle outputs."""
    rows, cols = x.shape
    G = len(off) - 1
    k_cap = mx.mx_grouped_k_capacity(rows, G)
    xb = mxsynth.bits(x)
    oqt, ost, opad = _grouped_oracle_par(xb, off, k_cap)
    qt = torch.full((cols, k_cap), 0xAB, dtype=torch.uint8, device="cuda")
    st_swz = torch.full((mx.mx_scale_swizzled_bytes(cols, k_cap // 32),), 0xCD, dtype=torch.uint8,
                        device="cuda")
    _, _, pad = mx.mx_quantize_colwise_grouped(x.cuda(), torch.from_numpy(off).cuda(), k_cap=k_cap,
                                               qt=qt, st_swz=st_swz)
    torch.cuda.synchronize()
    pad_h = pad.cpu().numpy()
    assert np.array_equal(pad_h, opad), f"{what}: pad offsets {pad_h} vs {opad}"
    pend = int(opad[-1])
    g = qt.cpu().numpy()
    bad = np.argwhere(g[:, :pend] != oqt[:, :pend])
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}"
    if sentinel:
        assert (g[:, pend:] == 0xAB).all(), f"{what}: columns past pad[G] were written"
    KT = k_cap // 256
    RT = (cols + 31) // 32
    swz = st_swz.cpu().numpy().reshape(RT, KT, 256)
    oswz = oracle.scale_swizzle(ost).reshape(RT, KT, 256)
    bad = np.argwhere(swz[:, :pend // 256] != oswz[:, :pend // 256])
    assert bad.size == 0, f"{what}: {len(bad)} rearranged scale bytes differ, first at {tuple(bad[0])}"
    if sentinel:
        assert (swz[:, pend // 256:] == 0xCD).all(), f"{what}: scale tiles past pad[G] were written"
    return qt, st_swz, pad, oqt, ost, opad


@pytest.mark.parametrize("sizes,cols", [
    ([37], 32),
    ([0, 37, 256, 300, 5], 64),
    ([0, 0, 0, 1], 288),
    ([513, 0, 255, 256, 257, 1, 0], 256),
    ([1000] * 3 + [0] * 5 + [31], 96),
])
def test_colwise_grouped_matches_oracle(gpu_lib, sizes, cols):
    off = _offsets(sizes)
    x = mxsynth.normal_bf16((int(off[-1]), cols), 1.0, seed=100 + len(sizes), outlier_frac=0.01, outlier_mul=100.0)
    _check_grouped_quant(gpu_lib, x, off, f"sizes={sizes} cols={cols}")


def test_colwise_grouped_no_rows(gpu_lib):
    """Every expert empty: each range is 256 zero columns with scale 0."""
    mx = gpu_lib
    off = np.zeros(4, np.int64)
    x = torch.zeros((1, 64), dtype=torch.bfloat16)[:0]
    qt, st_swz, pad = mx.mx_quantize_colwise_grouped(x.cuda(), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert pad.cpu().tolist() == [0, 256, 512, 768]
    assert (qt[:, :768].cpu() == 0).all()
    swz = st_swz.cpu().numpy().reshape(2, -1, 256)
    assert (swz[:, :3] == 0).all()


@pytest.mark.parametrize("sizes,M,N,dtype", [
    ([37], 32, 32, torch.bfloat16),
    ([0, 37, 256, 300, 5], 96, 224, torch.bfloat16),
    ([700, 0, 1, 513], 288, 256, torch.float32),
    ([100] * 9, 256, 512, torch.bfloat16),
    ([2000, 3, 0, 600], 64, 544, torch.float32),
])
def test_wgrad_matches_oracle(gpu_lib, sizes, M, N, dtype):
    mx = gpu_lib
    off = _offsets(sizes)
    T = int(off[-1])
    dy = mxsynth.normal_bf16((T, M), 1e-3, seed=200 + M, outlier_frac=0.01, outlier_mul=100.0)
    x = mxsynth.normal_bf16((T, N), 1.0, seed=300 + N, outlier_frac=0.01, outlier_mul=100.0)
    qa, sa_swz, pad, oqa, osa, opad = _check_grouped_quant(mx, dy, off, "dY", sentinel=False)
    qb, sb_swz, _, oqb, osb, _ = _check_grouped_quant(mx, x, off, "X", sentinel=False)
    C = mx.mx_grouped_gemm_wgrad(pad, qa, sa_swz, qb, sb_swz, out_dtype=dtype)
    torch.cuda.synchronize()
    assert C.shape == (len(sizes), M, N)
    r = wgrad_ref(opad, oqa, osa, oqb, osb)
    stats = assert_gemm_close(C, r, f"wgrad {sizes}")
    for g, m in enumerate(sizes):
        if m == 0:
            assert (C[g] == 0).all(), f"expert {g} has no rows but a nonzero gradient"
    print(stats_line(f"wgrad {sizes} {M}x{N}", stats))


def test_wgrad_repeatable_and_offsets_change_only_their_expert(gpu_lib):
    """Same inputs give the same bytes; moving rows between two experts
    changes only those two experts' gradients."""
    mx = gpu_lib
    sizes = [300, 200, 500, 24]
    off = _offsets(sizes)
    T, M, N = int(off[-1]), 128, 256
    dy = mxsynth.normal_bf16((T, M), 1e-3, seed=41).cuda()
    x = mxsynth.normal_bf16((T, N), 1.0, seed=42).cuda()

    def run(o):
        od = torch.from_numpy(o).cuda()
        qa, sa, pad = mx.mx_quantize_colwise_grouped(dy, od)
        qb, sb, _ = mx.mx_quantize_colwise_grouped(x, od)
        return mx.mx_grouped_gemm_wgrad(pad, qa, sa, qb, sb)

    c1, c2 = run(off), run(off)
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    off2 = off.copy()
    off2[2] += 64          # 64 rows move from expert 2 to expert 1
    c3 = run(off2)
    same = [torch.equal(c1[g].view(torch.int16), c3[g].view(torch.int16)) for g in range(4)]
    assert same == [True, False, False, True]


def test_moe_backward_qwen3_30b_a3b(gpu_lib):
    """Full size: 163840 routed rows over 128 experts with Zipf(1.1) loads.
    Per projection, the grouped column-wise quantization of dY and of the
    forward input (bytes exact over every column range), the weight gradient
    on sampled entries of every expert, and the data gradient through the
    column-wise expert weights on sampled rows of every expert."""
    mx = gpu_lib
    rows_per, a_gu, a_dn, w_gu, w_dn = mxsynth.moe_inputs()
    dy_gu, dy_dn = mxsynth.moe_bwd_grads()
    off = mxsynth.offsets_from_rows(rows_per)
    offd = torch.from_numpy(off).cuda()
    G = len(rows_per)
    rng = np.random.default_rng(6)
    # (name, dY [T][Nout], forward input X [T][Kin], W [G][Nout][Kin])
    for name, dy, x, w in (("gate_up", dy_gu, a_gu, w_gu), ("down", dy_dn, a_dn, w_dn)):
        print(f"moe bwd {name}: quantize", flush=True)
        qa, sa, pad, oqa, osa, opad = _check_grouped_quant(mx, dy, off, f"{name} dY", sentinel=False)
        qb, sb, _, oqb, osb, _ = _check_grouped_quant(mx, x, off, f"{name} X", sentinel=False)
        Nout, Kin = w.shape[1], w.shape[2]
        print(f"moe bwd {name}: wgrad {G}x{Nout}x{Kin}", flush=True)
        C = mx.mx_grouped_gemm_wgrad(pad, qa, sa, qb, sb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        # every 256 x 256 tile of every expert's gradient (lattice), plus its corners
        gs, rs, cs = lattice_wgrad(rng, G, Nout, Kin)
        gc = np.repeat(np.arange(G), 4)
        rc = np.tile([0, Nout - 1, 0, Nout - 1], G)
        cc = np.tile([0, Kin - 1, Kin - 1, 0], G)
        gs, rs, cs = np.concatenate([gs, gc]), np.concatenate([rs, rc]), np.concatenate([cs, cc])
        st = check_sampled_wgrad(C, gs, rs, cs, opad, oqa, osa, oqb, osb, f"{name} wgrad")
        print(stats_line(f"moe bwd {name} wgrad", st), flush=True)
        oqa_dy, oswz_dy = oqa, oracle.scale_swizzle(osa)
        del C, qa, sa, qb, sb, oqb

        # data gradient: dX = dY . W_g, B = column-wise W_g ([Kin][Nout] per expert)
        print(f"moe bwd {name}: dgrad", flush=True)
        _, _, wqt, wst_swz = mx.mx_quantize_dual_experts(w.cuda())
        wb = mxsynth.bits(w)
        parts = _pool_map(lambda g: oracle.quantize_colwise(wb[g]), range(G))
        owqt = np.stack([p[0] for p in parts])
        owst = np.stack([p[1] for p in parts])
        got_qt = wqt.cpu().numpy()
        assert np.array_equal(got_qt, owqt), f"{name}: column-wise expert weights differ"
        stb = mx.mx_scale_swizzled_bytes(Kin, Nout // 32)
        oswz = np.concatenate([oracle.scale_swizzle(owst[g]) for g in range(G)])
        assert np.array_equal(wst_swz.cpu().numpy(), oswz), f"{name}: expert weight scales differ"
        assert wst_swz.numel() == G * stb
        # dY row-wise and per-expert column-wise from one read
        dq, ds_swz, dqt, dst_swz, dpad = mx.mx_quantize_dual_grouped(dy.cuda(), offd)
        odq, ods = mxsynth_rowwise(dy)
        assert np.array_equal(dq.cpu().numpy(), odq), f"{name}: dual grouped row-wise codes differ"
        assert np.array_equal(ds_swz.cpu().numpy(), oracle.scale_swizzle(ods))
        assert np.array_equal(dpad.cpu().numpy(), opad)
        pend = int(opad[-1])
        assert np.array_equal(dqt.cpu().numpy()[:, :pend], oqa_dy[:, :pend]), \
            f"{name}: dual grouped column-wise codes differ"
        KT = dqt.shape[1] // 256
        assert np.array_equal(dst_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256],
                              oswz_dy.reshape(-1, KT, 256)[:, :pend // 256])
        del dqt, dst_swz
        D = mx.mx_grouped_gemm(offd, dq, ds_swz, wqt, wst_swz, out_dtype=torch.bfloat16)
        firsts = off[:-1][rows_per > 0]
        lasts = off[1:][rows_per > 0] - 1
        rl, cl = lattice_grouped(rng, off, Kin)
        rows = np.concatenate([rl, firsts, lasts, rng.integers(0, int(off[-1]), 512)])
        cols = np.concatenate([cl, rng.integers(0, Kin, rows.size - rl.size)])
        st = check_sampled_grouped(D, rows, cols, off, odq, ods, owqt, owst, f"{name} dgrad")
        print(stats_line(f"moe bwd {name} dgrad", st), flush=True)
        del D, dq, ds_swz, wqt, wst_swz, oqa_dy, oswz_dy


def mxsynth_rowwise(x):
    from gpu_util import oracle_rowwise_par
    return oracle_rowwise_par(mxsynth.bits(x))


def test_offsets_outside_the_stated_properties_stay_in_bounds(gpu_lib):
    """Offsets that are not nondecreasing within [0, rows] (and pad offsets
    that are not 256-aligned) give unspecified results but run to completion
    inside the buffers: the quantizer clamps the offsets into [0, rows] and
    makes the ranges nondecreasing, the GEMM clamps every range to at least
    one 256-column group inside [0, k_cap).  Checked here: both calls
    complete, the quantizer's ranges are 256-aligned, nondecreasing and end
    at most at k_cap, bytes past the buffers' ends are untouched, and the
    product is finite."""
    mx = gpu_lib
    rows, cols, G = 1000, 64, 4
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=55).cuda()
    off = torch.tensor([0, 500, 100, 5000, -7], dtype=torch.int64, device="cuda")
    k_cap = mx.mx_grouped_k_capacity(rows, G)
    guard = 4096
    qt_buf = torch.full((cols * k_cap + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    qt = qt_buf[:cols * k_cap].view(cols, k_cap)
    swz_n = mx.mx_scale_swizzled_bytes(cols, k_cap // 32)
    st_buf = torch.full((swz_n + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    _, _, pad = mx.mx_quantize_colwise_grouped(x, off, k_cap=k_cap, qt=qt, st_swz=st_buf[:swz_n])
    torch.cuda.synchronize()
    p = pad.cpu().numpy()
    assert p[0] == 0 and (np.diff(p) >= 0).all() and (p % 256 == 0).all() and p[-1] <= k_cap
    assert (qt_buf[cols * k_cap:].cpu() == 0x5A).all() and (st_buf[swz_n:].cpu() == 0x5A).all()
    # a product over ranges that are neither aligned nor ordered
    bad = torch.tensor([0, 300, 100, 10 ** 9, -256], dtype=torch.int64, device="cuda")
    c_buf = torch.full((G * cols * cols + guard,), 7.0, dtype=torch.float32, device="cuda")
    c = c_buf[:G * cols * cols].view(G, cols, cols)
    mx.mx_grouped_gemm_wgrad(bad, qt, st_buf[:swz_n], qt, st_buf[:swz_n], c=c)
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    assert (c_buf[G * cols * cols:] == 7.0).all()


@pytest.mark.parametrize("sizes,cols", [([37], 256), ([0, 37, 256, 300, 5], 512), ([513, 0, 255, 1, 31], 768)])
def test_dual_grouped_matches_oracle(gpu_lib, sizes, cols):
    """Row-wise (every row, scales rearranged) and per-expert column-wise
    quantization from one read: each output equals its oracle."""
    mx = gpu_lib
    off = _offsets(sizes)
    rows = int(off[-1])
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=600 + rows, outlier_frac=0.01, outlier_mul=100.0)
    xb = mxsynth.bits(x)
    q, s_swz, qt, st_swz, pad = mx.mx_quantize_dual_grouped(x.cuda(), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rowwise(xb)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(oracle.scale_unswizzle(s_swz.cpu().numpy(), rows, cols // 32), os_)
    k_cap = qt.shape[1]
    oqt, ost, opad = oracle.quantize_colwise_grouped(xb, off, k_cap)
    assert np.array_equal(pad.cpu().numpy(), opad)
    pend = int(opad[-1])
    assert np.array_equal(qt.cpu().numpy()[:, :pend], oqt[:, :pend])
    KT = k_cap // 256
    assert np.array_equal(st_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256],
                          oracle.scale_swizzle(ost).reshape(-1, KT, 256)[:, :pend // 256])


@pytest.mark.parametrize("sizes,F", [([37], 256), ([0, 37, 256, 300, 5], 512), ([513, 0, 255, 1, 31], 768),
                                     ([0, 0], 256)])
def test_swiglu_dual_grouped_matches_composition_and_oracle(gpu_lib, sizes, F):
    """h = SwiGLU(gate, up) quantized row-wise and per expert column-wise from
    one read of the gate/up output, h never written.  The result is byte-equal
    to mx_swiglu_quantize (its h and row-wise output) followed by
    mx_quantize_dual_grouped of that h.  Each output also equals the oracle's
    quantization of that h; h itself is pinned against the oracle's SwiGLU in
    tests/test_gpu_swiglu.py.  Gate values far out on both sides, zeros and
    negative zeros are planted."""
    mx = gpu_lib
    off = _offsets(sizes)
    rows = int(off[-1])
    gu = mxsynth.normal_bf16((rows, 2 * F), 1.0, seed=900 + rows + F, outlier_frac=0.01, outlier_mul=100.0)
    gb = mxsynth.bits(gu).copy()
    if rows:
        rng = np.random.default_rng(rows + F)
        for v in (0xC2C8, 0x4248, 0x0000, 0x8000, 0xC1A0, 0x42B2, 0xC2B2):   # -100, 50, 0, -0, -20, 89, -89
            gb[rng.integers(0, rows, 8), rng.integers(0, F, 8)] = v
    gu_d = mxsynth.from_bits(gb).cuda() if rows else torch.empty((0, 2 * F), dtype=torch.bfloat16, device="cuda")
    off_d = torch.from_numpy(off).cuda()
    q, s_swz, qt, st_swz, pad = mx.mx_swiglu_quantize_dual_grouped(gu_d, off_d)
    h = torch.empty((rows, F), dtype=torch.bfloat16, device="cuda")
    if rows:
        q1, s1, h = mx.mx_swiglu_quantize(gu_d, want_h=True)
    cq, cs, cqt, cst, cpad = mx.mx_quantize_dual_grouped(h, off_d)
    torch.cuda.synchronize()
    k_cap = qt.shape[1]
    assert k_cap == cqt.shape[1]
    assert torch.equal(pad, cpad)
    pend = int(pad[-1])
    KT = k_cap // 256
    assert torch.equal(qt[:, :pend], cqt[:, :pend])
    assert torch.equal(st_swz.view(-1, KT, 256)[:, :pend // 256], cst.view(-1, KT, 256)[:, :pend // 256])
    hb = mxsynth.bits(h.cpu())
    oqt, ost, opad = oracle.quantize_colwise_grouped(hb, off, k_cap)
    assert np.array_equal(pad.cpu().numpy(), opad)
    assert np.array_equal(qt.cpu().numpy()[:, :pend], oqt[:, :pend])
    assert np.array_equal(st_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256],
                          oracle.scale_swizzle(ost).reshape(-1, KT, 256)[:, :pend // 256])
    if rows:
        assert torch.equal(q, cq) and torch.equal(q, q1)
        us = oracle.scale_unswizzle(s_swz.cpu().numpy(), rows, F // 32)
        assert np.array_equal(us, oracle.scale_unswizzle(s1.cpu().numpy(), rows, F // 32))
        oq, os_ = oracle.quantize_rowwise(hb)
        assert np.array_equal(q.cpu().numpy(), oq)
        assert np.array_equal(us, os_)


@pytest.mark.parametrize("row_wise", [False, True])
def test_grouped_quantizers_strided_views(gpu_lib, row_wise):
    """x a column slice of a wider BF16 tensor (ld_x > cols), and the codes
    written into wider operands (ld_q > cols, ld_qt > k_cap): the quantizers
    address rows through the leading dimensions only, and leave the bytes
    around the views untouched.  The column-only case takes cols = 96, so
    the last 256-column tile has lanes past cols (they load and store
    nothing)."""
    mx = gpu_lib
    sizes = [300, 0, 37, 513, 1]
    off = _offsets(sizes)
    rows = int(off[-1])
    cols = 512 if row_wise else 96
    wide = mxsynth.normal_bf16((rows, cols + 192), 1.0, seed=700 + cols, outlier_frac=0.01,
                               outlier_mul=50.0).cuda()
    x = wide[:, 64:64 + cols]
    assert x.stride(0) == cols + 192
    xb = mxsynth.bits(x.cpu().contiguous())
    G = len(sizes)
    k_cap = mx.mx_grouped_k_capacity(rows, G)
    qt_wide = torch.full((cols, k_cap + 256), 0xAB, dtype=torch.uint8, device="cuda")
    qt = qt_wide[:, :k_cap]
    st_swz = torch.empty(mx.mx_scale_swizzled_bytes(cols, k_cap // 32), dtype=torch.uint8, device="cuda")
    offd = torch.from_numpy(off).cuda()
    if row_wise:
        q_wide = torch.full((rows, cols + 128), 0xEE, dtype=torch.uint8, device="cuda")
        q = q_wide[:, 128:]
        _, s_swz, _, _, pad = mx.mx_quantize_dual_grouped(x, offd, k_cap=k_cap, q=q, qt=qt, st_swz=st_swz)
    else:
        _, _, pad = mx.mx_quantize_colwise_grouped(x, offd, k_cap=k_cap, qt=qt, st_swz=st_swz)
    torch.cuda.synchronize()
    oqt, ost, opad = oracle.quantize_colwise_grouped(xb, off, k_cap)
    assert np.array_equal(pad.cpu().numpy(), opad)
    pend = int(opad[-1])
    g = qt_wide.cpu().numpy()
    assert np.array_equal(g[:, :pend], oqt[:, :pend])
    assert (g[:, k_cap:] == 0xAB).all(), "bytes past each qt row's k_cap were written"
    KT = k_cap // 256
    assert np.array_equal(st_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256],
                          oracle.scale_swizzle(ost).reshape(-1, KT, 256)[:, :pend // 256])
    if row_wise:
        oq, os_ = oracle.quantize_rowwise(xb)
        gq = q_wide.cpu().numpy()
        assert np.array_equal(gq[:, 128:], oq)
        assert (gq[:, :128] == 0xEE).all(), "bytes before each q row were written"
        assert np.array_equal(oracle.scale_unswizzle(s_swz.cpu().numpy(), rows, cols // 32), os_)
