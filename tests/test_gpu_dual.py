"""GPU parity of the fused dual-orientation quantizer (mx_quantize_dual).

Bar: bit-exact bytes.  Its four outputs must equal, byte for byte, the
oracle's row-wise codes, the oracle's column-wise (transposed) codes, and the
oracle's rearrangement of each of the two scale sets (the same pins as the
separate quantizers and the rearrangement)."""
import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import bf16_dev

pytestmark = pytest.mark.gpu


def _ref(x):
    oq, os_ = oracle.quantize_rowwise(x)
    oqt, ost = oracle.quantize_colwise(x)
    return oq, oracle.scale_swizzle(os_), oqt, oracle.scale_swizzle(ost)


def _eq(got, ref, what):
    g = got.cpu().numpy()
    bad = np.argwhere(g != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}"


def _check(mx, x, what):
    outs = mx.mx_quantize_dual(bf16_dev(mxsynth.from_bits(x)))
    for got, ref, name in zip(outs, _ref(x), ("q", "s_swz", "qt", "st_swz")):
        _eq(got, ref, f"{what} {name}")


@pytest.mark.parametrize("rows,cols", [(32, 32), (64, 96), (256, 256), (288, 320), (512, 1056),
                                       (4096, 4096),
                                       # 32+ tiles across: the per-XCD tile order, padded grid
                                       (1184, 8224), (320, 16384)])
def test_dual_matches_oracle(gpu_lib, rows, cols):
    x = mxsynth.bits(mxsynth.normal_bf16((rows, cols), 1e-3, rows * 7 + cols, 0.01, 50.0))
    _check(gpu_lib, x, f"{rows}x{cols}")


def test_dual_special_values(gpu_lib):
    """Every magnitude pattern as a block maximum in one orientation (NaN and Inf
    included), and scattered NaN/Inf that poison blocks of both orientations."""
    p = np.arange(0x8000, dtype=np.int64)
    i = np.arange(32, dtype=np.int64)
    blocks = (p[:, None] * i[None, :]) // 32
    blocks[p, p % 32] = p
    sign = ((p[:, None] + i[None, :]) & 1) << 15
    x = ((blocks | sign).astype(np.uint16)).reshape(512, 2048)
    x[5, 77] = 0x7FC0
    x[300, 1000] = 0xFF80
    _check(gpu_lib, x, "special")


def test_dual_equals_separate_kernels(gpu_lib):
    mx = gpu_lib
    x = bf16_dev(mxsynth.normal_bf16((768, 1280), 1.0, 11))
    q, s_swz, qt, st_swz = mx.mx_quantize_dual(x)
    q1, s1 = mx.mx_quantize_rowwise(x)
    qt1, st1 = mx.mx_quantize_colwise(x)
    assert torch.equal(q, q1) and torch.equal(qt, qt1)
    assert torch.equal(s_swz, mx.mx_scale_swizzle(s1))
    assert torch.equal(st_swz, mx.mx_scale_swizzle(st1))


def test_dual_into_concatenated_operands(gpu_lib):
    """Two weights stacked along rows for the forward operand (row-wise scales at
    a tile-row offset) and side by side along K for the backward operand
    (column-wise scales at a 256-K-group offset), as for a fused gate/up
    projection: the result equals the quantization of the stacked tensor."""
    mx = gpu_lib
    R1, R2, C = 768, 512, 544
    x1 = mxsynth.bits(mxsynth.normal_bf16((R1, C), 1.0, 21))
    x2 = mxsynth.bits(mxsynth.normal_bf16((R2, C), 3.0, 22))
    R = R1 + R2
    dev = "cuda"
    q = torch.empty((R, C), dtype=torch.uint8, device=dev)
    qt = torch.empty((C, R), dtype=torch.uint8, device=dev)
    s_swz = torch.full((mx.mx_scale_swizzled_bytes(R, C // 32),), 0xEE, dtype=torch.uint8, device=dev)
    st_swz = torch.full((mx.mx_scale_swizzled_bytes(C, R // 32),), 0xEE, dtype=torch.uint8, device=dev)
    kts, ktst = (C // 32 + 7) // 8, (R // 32 + 7) // 8
    mx.mx_quantize_dual(bf16_dev(mxsynth.from_bits(x1)), q=q[:R1], s_swz=s_swz, qt=qt[:, :R1],
                        st_swz=st_swz, s_tiles=kts, st_tiles=ktst)
    mx.mx_quantize_dual(bf16_dev(mxsynth.from_bits(x2)), q=q[R1:],
                        s_swz=s_swz[(R1 // 32) * kts * 256:], qt=qt[:, R1:],
                        st_swz=st_swz[(R1 // 256) * 256:], s_tiles=kts, st_tiles=ktst)
    for got, ref, name in zip((q, s_swz, qt, st_swz), _ref(np.concatenate([x1, x2], 0)),
                              ("q", "s_swz", "qt", "st_swz")):
        _eq(got, ref, f"stacked {name}")


def test_dual_batch_matches_oracle(gpu_lib):
    """A layer's worth of jobs in one launch: different shapes (one of them wide
    enough for the per-XCD tile order, one a quarter of the chip), two of them
    writing the halves of stacked and side-by-side operands, and an empty job."""
    mx = gpu_lib
    dev = "cuda"
    shapes = {"a": (256, 512), "b": (1024, 256), "c": (96, 8224), "g": (512, 288), "u": (256, 288)}
    X = {k: mxsynth.bits(mxsynth.normal_bf16(v, 1.0 + i, 40 + i)) for i, (k, v) in enumerate(shapes.items())}
    outs = {}
    jobs = []
    for k in ("a", "b", "c"):
        r, c = shapes[k]
        o = dict(x=bf16_dev(mxsynth.from_bits(X[k])),
                 q=torch.empty((r, c), dtype=torch.uint8, device=dev),
                 s_swz=torch.empty((mx.mx_scale_swizzled_bytes(r, c // 32),), dtype=torch.uint8, device=dev),
                 qt=torch.empty((c, r), dtype=torch.uint8, device=dev),
                 st_swz=torch.empty((mx.mx_scale_swizzled_bytes(c, r // 32),), dtype=torch.uint8, device=dev))
        outs[k] = o
        jobs.append(o)
    # g and u: stacked rows (forward operand), side by side along K (backward operand)
    R, C = 512 + 256, 288
    kts, ktst = (C // 32 + 7) // 8, (R // 32 + 7) // 8
    fused = dict(q=torch.empty((R, C), dtype=torch.uint8, device=dev),
                 s_swz=torch.full((mx.mx_scale_swizzled_bytes(R, C // 32),), 0xEE, dtype=torch.uint8, device=dev),
                 qt=torch.empty((C, R), dtype=torch.uint8, device=dev),
                 st_swz=torch.full((mx.mx_scale_swizzled_bytes(C, R // 32),), 0xEE, dtype=torch.uint8, device=dev))
    for k, r0, r1 in (("g", 0, 512), ("u", 512, 768)):
        jobs.append(dict(x=bf16_dev(mxsynth.from_bits(X[k])), q=fused["q"][r0:r1],
                         s_swz=fused["s_swz"][(r0 // 32) * kts * 256:], s_tiles=kts,
                         qt=fused["qt"][:, r0:r1], st_swz=fused["st_swz"][(r0 // 256) * 256:],
                         st_tiles=ktst))
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    jobs.append(dict(x=e, q=torch.empty((0, 64), dtype=torch.uint8, device=dev),
                     s_swz=torch.empty((4,), dtype=torch.uint8, device=dev),
                     qt=torch.empty((64, 0), dtype=torch.uint8, device=dev),
                     st_swz=torch.empty((4,), dtype=torch.uint8, device=dev)))
    mx.mx_quantize_dual_batch(jobs)
    for k in ("a", "b", "c"):
        o = outs[k]
        for got, ref, name in zip((o["q"], o["s_swz"], o["qt"], o["st_swz"]), _ref(X[k]),
                                  ("q", "s_swz", "qt", "st_swz")):
            _eq(got, ref, f"batch {k} {name}")
    for got, ref, name in zip((fused["q"], fused["s_swz"], fused["qt"], fused["st_swz"]),
                              _ref(np.concatenate([X["g"], X["u"]], 0)),
                              ("q", "s_swz", "qt", "st_swz")):
        _eq(got, ref, f"batch stacked {name}")


@pytest.mark.parametrize("G,rows,cols", [(1, 32, 32), (5, 96, 64), (3, 288, 320), (2, 256, 8224),
                                         (17, 1536, 256)])
def test_dual_experts_matches_oracle(gpu_lib, G, rows, cols):
    """Stacked expert weights in one launch: every expert's four outputs equal
    the oracle's, at the expert's place in each stack."""
    mx = gpu_lib
    w = mxsynth.normal_bf16((G, rows, cols), 0.02, seed=900 + G, outlier_frac=0.001, outlier_mul=20.0)
    q, s_swz, qt, st_swz = mx.mx_quantize_dual_experts(w.cuda())
    torch.cuda.synchronize()
    sb = mx.mx_scale_swizzled_bytes(rows, cols // 32)
    stb = mx.mx_scale_swizzled_bytes(cols, rows // 32)
    assert s_swz.numel() == G * sb and st_swz.numel() == G * stb
    for g in range(G):
        oq, os_swz, oqt, ost_swz = _ref(mxsynth.bits(w[g]))
        _eq(q[g], oq, f"expert {g} q")
        _eq(s_swz[g * sb:(g + 1) * sb], os_swz, f"expert {g} s_swz")
        _eq(qt[g], oqt, f"expert {g} qt")
        _eq(st_swz[g * stb:(g + 1) * stb], ost_swz, f"expert {g} st_swz")
