"""GPU parity of the quantizers and the scale rearrangement against the oracle.

Bar: bit-exact bytes (codes and scales), every byte of every output.  The
E4M3/E8M0 rule is the one pinned in tests/test_oracle_pins.py.
"""
import os

import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import bf16_dev, to_dev

pytestmark = pytest.mark.gpu


def _golden_x():
    from test_oracle_pins import GOLDEN_BLOCKS
    return np.array([b["x"] for b in GOLDEN_BLOCKS], np.uint16)


def test_golden_blocks_rowwise_and_colwise(gpu_lib):
    mx = gpu_lib
    x = _golden_x()  # [7][32]
    xt = mxsynth.from_bits(x)
    q, s = mx.mx_quantize_rowwise(bf16_dev(xt))
    oq, os_ = oracle.quantize_rowwise(x)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy(), os_)
    # the same blocks down columns: x^T is [32][7] -> pad columns to a multiple of 8
    xc = np.zeros((32, 8), np.uint16)
    xc[:, :7] = x.T
    qt, st = mx.mx_quantize_colwise(bf16_dev(mxsynth.from_bits(xc)))
    oqt, ost = oracle.quantize_colwise(xc)
    assert np.array_equal(qt.cpu().numpy(), oqt) and np.array_equal(st.cpu().numpy(), ost)


def _exhaustive_blocks():
    """Blocks whose first element fixes the scale code c (amax = largest BF16 of
    binade c + 8, or of binade <= 8 for c = 0) and whose other 31 elements run
    over every finite BF16 of magnitude <= amax, both signs: every (element,
    scale) pair the quantizer can meet."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[((allb >> 7) & 0xFF) != 0xFF]
    mag = fin & 0x7FFF
    rows = []
    for c in range(0, 247):
        e_amax = c + 8
        amax = np.uint16((e_amax << 7) | 0x7F)
        els = fin[mag <= amax]
        n = (els.size + 30) // 31
        pad = np.zeros(n * 31, np.uint16)
        pad[:els.size] = els
        blk = np.concatenate([np.full((n, 1), amax, np.uint16), pad.reshape(n, 31)], axis=1)
        rows.append(blk)
    return np.concatenate(rows, 0)


def _assert_codes(got: torch.Tensor, ref: np.ndarray, x: np.ndarray, what: str):
    g = got.cpu().numpy()
    bad = np.argwhere(g != ref)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"x={x[tuple(bad[0])]:#06x} got {g[tuple(bad[0])]:#04x} "
                           f"ref {ref[tuple(bad[0])]:#04x}")


def _blocks_to_matrix(blocks: np.ndarray) -> np.ndarray:
    """[nblk][32] -> [R][2048] (64 blocks per row, R a multiple of 8, zero padded)."""
    nblk = blocks.shape[0]
    R = -(-nblk // 64)
    R = -(-R // 8) * 8
    x = np.zeros((R * 64, 32), np.uint16)
    x[:nblk] = blocks
    return x.reshape(R, 2048)


def _check_both_orientations(mx, x: np.ndarray, what: str):
    """Row-wise on x, and column-wise on x^T, whose column blocks are the row blocks of x."""
    q, s = mx.mx_quantize_rowwise(bf16_dev(mxsynth.from_bits(x)))
    oq, os_ = oracle.quantize_rowwise(x)
    _assert_codes(q, oq, x, what + " rowwise codes")
    _assert_codes(s, os_, np.zeros_like(os_, np.uint16), what + " rowwise scales")
    xt = np.ascontiguousarray(x.T)
    qt, st = mx.mx_quantize_colwise(bf16_dev(mxsynth.from_bits(xt)))
    oqt, ost = oracle.quantize_colwise(xt)
    _assert_codes(qt, oqt, x, what + " colwise codes")
    _assert_codes(st, ost, np.zeros_like(ost, np.uint16), what + " colwise scales")
    return os_


def test_exhaustive_encoder_table_on_device(gpu_lib):
    """All reachable (BF16 element, scale code) pairs, ~9 M elements, both kernels."""
    x = _blocks_to_matrix(_exhaustive_blocks())
    os_ = _check_both_orientations(gpu_lib, x, "exhaustive")
    assert set(np.unique(os_).tolist()) == set(range(0, 247))


def test_every_block_maximum(gpu_lib):
    """Every magnitude pattern 0..0x7FFF as a block maximum (NaN and Inf included),
    at a position and sign that vary with the pattern; the other elements are
    smaller magnitudes of alternating sign."""
    p = np.arange(0x8000, dtype=np.int64)
    i = np.arange(32, dtype=np.int64)
    blocks = (p[:, None] * i[None, :]) // 32                       # magnitudes below p
    blocks[p, p % 32] = p                                          # the maximum itself
    sign = ((p[:, None] + i[None, :]) & 1) << 15
    x = _blocks_to_matrix((blocks | sign).astype(np.uint16))
    os_ = _check_both_orientations(gpu_lib, x, "block maxima")
    assert (os_ == 0xFF).sum() == 0x8000 - 0x7F80                  # every Inf/NaN block
    assert (os_ == 0).sum() >= 8 << 7                              # all tiny maxima clamp to 0


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (128, 256), (257, 4096), (33, 12288)])
def test_rowwise_shapes(gpu_lib, rows, cols):
    mx = gpu_lib
    x = mxsynth.normal_bf16((rows, cols), 1.0, rows * 7 + cols, 0.01, 100.0)
    q, s = mx.mx_quantize_rowwise(bf16_dev(x))
    oq, os_ = oracle.quantize_rowwise(mxsynth.bits(x))
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)


def test_rowwise_strided_and_byte_views(gpu_lib):
    """Leading dimensions larger than the row (a column slice of a wider tensor)."""
    mx = gpu_lib
    big = mxsynth.normal_bf16((40, 512), 0.02, 11, 0.001, 20.0)
    xs = bf16_dev(big)[:, 128:384]                     # ld_x = 512
    qbuf = torch.full((40, 320), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((40, 12), 0xCD, dtype=torch.uint8, device="cuda")
    q, s = mx.mx_quantize_rowwise(xs, q=qbuf[:, :256], s=sbuf[:, :8])
    oq, os_ = oracle.quantize_rowwise(mxsynth.bits(big[:, 128:384].contiguous()))
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    # bytes outside the used window are untouched
    assert (qbuf[:, 256:] == 0xAB).all() and (sbuf[:, 8:] == 0xCD).all()


@pytest.mark.parametrize("rows,cols", [(32, 8), (64, 24), (128, 256), (160, 264), (4096, 1024),
                                       (96, 4104),
                                       # 32+ column tiles: the grouped, per-XCD tile order, with
                                       # a ragged last tile-row group and a grid padded to 8
                                       (1184, 8200), (4224, 8192), (32, 16384)])
def test_colwise_shapes(gpu_lib, rows, cols):
    mx = gpu_lib
    x = mxsynth.normal_bf16((rows, cols), 1e-3, rows * 13 + cols, 0.01, 50.0)
    qt, st = mx.mx_quantize_colwise(bf16_dev(x))
    oqt, ost = oracle.quantize_colwise(mxsynth.bits(x))
    assert np.array_equal(qt.cpu().numpy(), oqt) and np.array_equal(st.cpu().numpy(), ost)


def test_colwise_strided_output(gpu_lib):
    mx = gpu_lib
    x = mxsynth.normal_bf16((64, 48), 1.0, 5)
    qbuf = torch.full((48, 80), 0x11, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((48, 5), 0x22, dtype=torch.uint8, device="cuda")
    qt, st = mx.mx_quantize_colwise(bf16_dev(x), qt=qbuf[:, :64], st_=sbuf[:, :2])
    oqt, ost = oracle.quantize_colwise(mxsynth.bits(x))
    assert np.array_equal(qt.cpu().numpy(), oqt) and np.array_equal(st.cpu().numpy(), ost)
    assert (qbuf[:, 64:] == 0x11).all() and (sbuf[:, 2:] == 0x22).all()


def test_tiny_config_bytes(gpu_lib):
    mx = gpu_lib
    A, B = mxsynth.tiny()
    qa, sa = mx.mx_quantize_rowwise(bf16_dev(A))
    qbt, sbt = mx.mx_quantize_colwise(bf16_dev(B))
    oqa, osa = oracle.quantize_rowwise(mxsynth.bits(A))
    oqb, osb = oracle.quantize_colwise(mxsynth.bits(B))
    for g, o in ((qa, oqa), (sa, osa), (qbt, oqb), (sbt, osb)):
        assert np.array_equal(g.cpu().numpy(), o)


def test_determinism_repeat_calls(gpu_lib):
    """Byte-for-byte: the same weights quantize to the same bytes on every call."""
    mx = gpu_lib
    w = bf16_dev(mxsynth.normal_bf16((1024, 4096), 0.02, 77, 0.001, 20.0))
    q1, s1 = mx.mx_quantize_rowwise(w)
    t1, u1 = mx.mx_quantize_colwise(w)
    for _ in range(3):
        q2, s2 = mx.mx_quantize_rowwise(w)
        t2, u2 = mx.mx_quantize_colwise(w)
        assert torch.equal(q1, q2) and torch.equal(s1, s2)
        assert torch.equal(t1, t2) and torch.equal(u1, u2)


def test_nan_inf_blocks(gpu_lib):
    mx = gpu_lib
    x = mxsynth.bits(mxsynth.normal_bf16((64, 64), 1.0, 3))
    x[3, 5] = 0x7FC0   # NaN
    x[40, 33] = 0xFF80  # -Inf
    x[10, 40] = 0x7F80  # +Inf
    xt = bf16_dev(mxsynth.from_bits(x))
    q, s = mx.mx_quantize_rowwise(xt)
    oq, os_ = oracle.quantize_rowwise(x)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    qt, st = mx.mx_quantize_colwise(xt)
    oqt, ost = oracle.quantize_colwise(x)
    assert np.array_equal(qt.cpu().numpy(), oqt) and np.array_equal(st.cpu().numpy(), ost)
    assert (os_ == 0xFF).sum() == 3


# ---------------------------------------------------------------------------
# scale rearrangement


@pytest.mark.parametrize("rows,kb", [(1, 1), (32, 8), (33, 9), (128, 8), (100, 24), (4096, 384),
                                     (4101, 77)])
def test_swizzle_matches_oracle(gpu_lib, rows, kb):
    mx = gpu_lib
    rng = np.random.default_rng(rows * 31 + kb)
    s = rng.integers(0, 255, size=(rows, kb), dtype=np.uint8)
    out = mx.mx_scale_swizzle(to_dev(s))
    assert np.array_equal(out.cpu().numpy(), oracle.scale_swizzle(s))


def test_swizzle_strided_input(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(9)
    s = rng.integers(0, 255, size=(70, 40), dtype=np.uint8)
    out = mx.mx_scale_swizzle(to_dev(s)[:, 3:30])
    assert np.array_equal(out.cpu().numpy(), oracle.scale_swizzle(s[:, 3:30].copy()))


@pytest.mark.parametrize("rows,cols", [(32, 256), (37, 512), (4608, 4096), (1000, 12288), (163840, 768)])
def test_rowwise_swz_matches_oracle(gpu_lib, rows, cols):
    """Row-wise codes and the rearranged scales in one pass: the codes equal
    the oracle's, every written scale byte sits where the oracle's
    rearrangement puts it (rows past the tensor in the last 32-row tile are
    padding the call does not write)."""
    import mxsynth
    mx = gpu_lib
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=rows + cols, outlier_frac=0.005, outlier_mul=50.0)
    xb = mxsynth.bits(x)
    q, s_swz = mx.mx_quantize_rowwise_swz(x.cuda())
    torch.cuda.synchronize()
    from gpu_util import oracle_rowwise_par
    oq, os_ = oracle_rowwise_par(xb)
    assert np.array_equal(q.cpu().numpy(), oq)
    got = s_swz.cpu().numpy()
    if rows % 32 == 0:
        assert np.array_equal(got, oracle.scale_swizzle(os_))
    else:
        assert np.array_equal(oracle.scale_unswizzle(got, rows, cols // 32), os_)


def test_rowwise_swz_into_larger_operand(gpu_lib):
    """Two tensors side by side along K (s_tiles of the larger operand): the
    result equals quantizing the concatenation."""
    import mxsynth
    mx = gpu_lib
    a = mxsynth.normal_bf16((64, 512), 1.0, seed=5)
    b = mxsynth.normal_bf16((64, 256), 1.0, seed=6)
    cat = torch.cat([a, b], dim=1)
    kt = 768 // 256
    q = torch.empty(64, 768, dtype=torch.uint8, device="cuda")
    s_swz = torch.full((mx.mx_scale_swizzled_bytes(64, 24),), 0xEE, dtype=torch.uint8, device="cuda")
    mx.mx_quantize_rowwise_swz(a.cuda(), q=q[:, :512], s_swz=s_swz, s_tiles=kt)
    mx.mx_quantize_rowwise_swz(b.cuda(), q=q[:, 512:], s_swz=s_swz[2 * 256:], s_tiles=kt)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rowwise(mxsynth.bits(cat))
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s_swz.cpu().numpy(), oracle.scale_swizzle(os_))


@pytest.mark.parametrize("rows,cols", [(256, 32), (512, 96), (768, 264 + 8 * 3),
                                       (4096, 1024), (4608, 4096),
                                       # 32+ column tiles (the per-XCD tile order), a ragged
                                       # last column tile and tile-row group
                                       (1280, 8192), (256, 16416)])
def test_colwise_swz_matches_oracle(gpu_lib, rows, cols):
    """Column-wise codes and the rearranged scales in one pass: the codes
    equal the oracle's column-wise codes and the scale buffer equals the
    oracle's rearrangement of its column-wise scales, every byte."""
    mx = gpu_lib
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=3 * rows + cols, outlier_frac=0.005, outlier_mul=50.0)
    qt, st_swz = mx.mx_quantize_colwise_swz(bf16_dev(x))
    torch.cuda.synchronize()
    from gpu_util import oracle_colwise_par
    oqt, ost = oracle_colwise_par(mxsynth.bits(x))
    assert np.array_equal(qt.cpu().numpy(), oqt)
    assert st_swz.numel() == mx.mx_scale_swizzled_bytes(cols, rows // 32)
    assert np.array_equal(st_swz.cpu().numpy(), oracle.scale_swizzle(ost))


def test_colwise_swz_strided_and_into_larger_operand(gpu_lib):
    """A strided input, and two tensors stacked along K (= their rows) written
    into one operand with st_tiles of the larger K: the result equals the
    column-wise quantization of the stacked tensor; bytes past the codes'
    columns are untouched."""
    mx = gpu_lib
    a = mxsynth.normal_bf16((256, 96), 1.0, seed=11)
    b = mxsynth.normal_bf16((512, 96), 2.0, seed=12)
    cat = torch.cat([a, b], dim=0)
    xbuf = torch.zeros(512, 136, dtype=torch.bfloat16, device="cuda")
    xbuf[:, :96] = b.cuda()
    kt = 768 // 256
    qbuf = torch.full((96, 800), 0x11, dtype=torch.uint8, device="cuda")
    st_swz = torch.full((mx.mx_scale_swizzled_bytes(96, 24),), 0xEE, dtype=torch.uint8, device="cuda")
    mx.mx_quantize_colwise_swz(a.cuda(), qt=qbuf[:, :256], st_swz=st_swz, st_tiles=kt)
    mx.mx_quantize_colwise_swz(xbuf[:, :96], qt=qbuf[:, 256:768], st_swz=st_swz[256:], st_tiles=kt)
    torch.cuda.synchronize()
    oqt, ost = oracle.quantize_colwise(mxsynth.bits(cat))
    assert np.array_equal(qbuf[:, :768].cpu().numpy(), oqt)
    assert (qbuf[:, 768:] == 0x11).all()
    assert np.array_equal(st_swz.cpu().numpy(), oracle.scale_swizzle(ost))


def _rowwise_swz_ref(x: torch.Tensor):
    """Oracle codes and scale buffer of mx_quantize_rowwise_swz (rows past the
    tensor in its last 32-row tile excepted: compared through unswizzle)."""
    from gpu_util import oracle_rowwise_par
    return oracle_rowwise_par(mxsynth.bits(x))


def _check_rowwise_swz(q: torch.Tensor, s_swz: torch.Tensor, x: torch.Tensor):
    rows, cols = x.shape
    oq, os_ = _rowwise_swz_ref(x)
    assert np.array_equal(q.cpu().numpy(), oq)
    got = s_swz.cpu().numpy()
    if rows % 32 == 0:
        assert np.array_equal(got, oracle.scale_swizzle(os_))
    else:
        assert np.array_equal(oracle.scale_unswizzle(got, rows, cols // 32), os_)


def test_rowwise_swz_batch_layer_activations(gpu_lib):
    """The two activations of a dense layer's forward products (4608 tokens:
    hidden 4096, intermediate 12288) in one launch, every byte against the
    oracle."""
    mx = gpu_lib
    xs = [mxsynth.normal_bf16((4608, 4096), 1.0, seed=21, outlier_frac=0.005, outlier_mul=50.0),
          mxsynth.normal_bf16((4608, 12288), 0.5, seed=22, outlier_frac=0.005, outlier_mul=50.0)]
    jobs = []
    for x in xs:
        r, c = x.shape
        jobs.append({"x": bf16_dev(x), "q": torch.empty(r, c, dtype=torch.uint8, device="cuda"),
                     "s_swz": torch.full((mx.mx_scale_swizzled_bytes(r, c // 32),), 0xEE, dtype=torch.uint8,
                                         device="cuda")})
    mx.mx_quantize_rowwise_swz_batch(jobs)
    torch.cuda.synchronize()
    for x, j in zip(xs, jobs):
        _check_rowwise_swz(j["q"], j["s_swz"], x)


def test_rowwise_swz_batch_ragged_jobs(gpu_lib):
    """Eight jobs of mixed, ragged shapes (one empty, one strided, two writing
    side by side into one operand), each equal to the oracle."""
    mx = gpu_lib
    shapes = [(37, 512), (0, 256), (256, 768), (1, 256), (1000, 4096), (33, 12288)]
    xs = [mxsynth.normal_bf16(s, 1.0, seed=40 + i, outlier_frac=0.01, outlier_mul=50.0)
          for i, s in enumerate(shapes)]
    jobs = []
    for x in xs:
        r, c = x.shape
        jobs.append({"x": bf16_dev(x), "q": torch.empty(r, c, dtype=torch.uint8, device="cuda"),
                     "s_swz": torch.full((max(mx.mx_scale_swizzled_bytes(r, c // 32), 1),), 0xEE,
                                         dtype=torch.uint8, device="cuda")})
    # the strided one: job 2 reads a view of a wider buffer and writes into a wider q
    xbuf = torch.zeros(256, 1024, dtype=torch.bfloat16, device="cuda")
    xbuf[:, :768] = xs[2].cuda()
    qbuf = torch.full((256, 1024), 0x11, dtype=torch.uint8, device="cuda")
    jobs[2]["x"], jobs[2]["q"] = xbuf[:, :768], qbuf[:, :768]
    # two halves of one [64][768] operand along K
    a = mxsynth.normal_bf16((64, 512), 1.0, seed=50)
    b = mxsynth.normal_bf16((64, 256), 1.0, seed=51)
    cat = torch.cat([a, b], dim=1)
    qc = torch.empty(64, 768, dtype=torch.uint8, device="cuda")
    sc = torch.full((mx.mx_scale_swizzled_bytes(64, 24),), 0xEE, dtype=torch.uint8, device="cuda")
    jobs.append({"x": a.cuda(), "q": qc[:, :512], "s_swz": sc, "s_tiles": 3})
    jobs.append({"x": b.cuda(), "q": qc[:, 512:], "s_swz": sc[512:], "s_tiles": 3})
    assert len(jobs) == 8
    mx.mx_quantize_rowwise_swz_batch(jobs)
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        if x.shape[0] == 0:
            continue
        _check_rowwise_swz(jobs[i]["q"], jobs[i]["s_swz"], x)
    assert (qbuf[:, 768:] == 0x11).all()
    _check_rowwise_swz(qc, sc, cat)
