"""CPU checks of the C ABI: the library loads without a GPU, exports every
declared entry point, and rejects invalid arguments before touching HIP.

No call here reaches a kernel: every call is either a host-only query or an
argument error (fake non-null pointers are never dereferenced, because
validation returns first).
"""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_08_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

FAKE = 0x10000  # 64 KiB-aligned fake device address; never dereferenced
FAKE2 = 0x40000000
FAKE3 = 0x80000000
FAKE4 = 0xC0000000
STREAM = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = mx.load()
    names = declared_functions()
    assert {"mx_quantize_rowwise", "mx_quantize_colwise", "mx_scale_swizzle", "mx_gemm",
            "mx_grouped_gemm", "mx_scale_swizzled_bytes", "mx_quantize_dual"} <= set(names)
    raw = ctypes.CDLL(mx.lib_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in include/mxfp8.h but not exported"
        assert hasattr(mx, n), f"{n} has no Python binding of the same name"
    assert L.mx_abi_version() == 9


def test_status_strings():
    L = mx.load()
    for code, name in [(0, "MX_OK"), (1, "MX_ERR_INVALID_ARG"), (2, "MX_ERR_SHAPE"),
                       (3, "MX_ERR_ALIGN"), (4, "MX_ERR_OVERLAP"), (5, "MX_ERR_UNSUPPORTED"),
                       (6, "MX_ERR_HIP")]:
        assert L.mx_status_string(code).decode() == name
    assert L.mx_status_string(99).decode() == "MX_ERR_UNKNOWN"


@pytest.mark.parametrize("rows,kb", [(0, 8), (1, 1), (32, 8), (33, 9), (4096, 128), (163840, 64),
                                     (12288, 768)])
def test_swizzled_bytes(rows, kb):
    expect = 0 if rows == 0 else ((rows + 31) // 32) * ((kb + 7) // 8) * 256
    assert mx.mx_scale_swizzled_bytes(rows, kb) == expect


def _err(L):
    return L.mx_last_error().decode()


def test_quantize_rowwise_validation():
    L = mx.load()
    f = L.mx_quantize_rowwise
    assert f(FAKE, 4, 48, 48, FAKE2, 48, FAKE3, 2, STREAM) == mx.MX_ERR_SHAPE
    assert "cols=48" in _err(L)
    assert f(FAKE, -1, 64, 64, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 32, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 64, FAKE2, 64, FAKE3, 1, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(0, 4, 64, 64, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE + 2, 4, 64, 64, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 4, 64, 68, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 4, 64, 64, FAKE2, 72, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    # q inside x
    assert f(FAKE, 4, 64, 64, FAKE + 64, 64, FAKE3, 2, STREAM) == mx.MX_ERR_OVERLAP
    # s inside q
    assert f(FAKE, 4, 64, 64, FAKE2, 64, FAKE2 + 100, 2, STREAM) == mx.MX_ERR_OVERLAP
    # empty problems are a no-op that succeeds (nothing launched)
    assert f(FAKE, 0, 64, 64, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_OK
    assert f(FAKE, 7, 0, 0, FAKE2, 0, FAKE3, 0, STREAM) == mx.MX_OK


def test_quantize_colwise_validation():
    L = mx.load()
    f = L.mx_quantize_colwise
    assert f(FAKE, 48, 64, 64, FAKE2, 48, FAKE3, 1, STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE, 64, 60, 64, FAKE2, 64, FAKE3, 2, STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE, 64, 64, 64, FAKE2, 32, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 64, 64, 64, FAKE2, 64, FAKE3, 1, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 64, 64, 64, FAKE2 + 8, 64, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 64, 64, 64, FAKE + 4096, 64, FAKE3, 2, STREAM) == mx.MX_ERR_OVERLAP
    assert f(FAKE, 0, 64, 64, FAKE2, 0, FAKE3, 0, STREAM) == mx.MX_OK


def test_quantize_dual_validation():
    L = mx.load()
    f = L.mx_quantize_dual
    FAKE5, FAKE6 = 0x100000000, 0x140000000
    # x[64][64]: q at FAKE2, s_swz at FAKE3 (2 tiles), qt at FAKE5, st_swz at FAKE6 (2 tiles)
    good = [FAKE, 64, 64, 64, FAKE2, 64, FAKE3, 1, FAKE5, 64, FAKE6, 1, STREAM]

    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a1=48) == mx.MX_ERR_SHAPE           # rows % 32
    assert call(a2=48, a3=48, a5=48) == mx.MX_ERR_SHAPE  # cols % 32
    assert call(a1=-32) == mx.MX_ERR_INVALID_ARG
    assert call(a3=32) == mx.MX_ERR_INVALID_ARG      # ld_x < cols
    assert call(a5=32) == mx.MX_ERR_INVALID_ARG      # ld_q < cols
    assert call(a9=32) == mx.MX_ERR_INVALID_ARG      # ld_qt < rows
    assert call(a2=512, a3=512, a5=512, a7=1) == mx.MX_ERR_INVALID_ARG  # s_tiles < ceil(512/256)
    assert call(a1=512, a9=512, a11=1) == mx.MX_ERR_INVALID_ARG         # st_tiles < ceil(512/256)
    assert "tiles" in _err(L)
    assert call(a4=0) == mx.MX_ERR_INVALID_ARG       # null q
    assert call(a0=FAKE + 2) == mx.MX_ERR_ALIGN
    assert call(a8=FAKE5 + 8) == mx.MX_ERR_ALIGN
    assert call(a6=FAKE3 + 2) == mx.MX_ERR_ALIGN
    assert call(a9=72) == mx.MX_ERR_ALIGN            # ld_qt % 16
    assert call(a4=FAKE + 128) == mx.MX_ERR_OVERLAP  # q inside x
    assert call(a10=FAKE5 + 256) == mx.MX_ERR_OVERLAP  # st_swz inside qt
    assert call(a6=FAKE2 + 64) == mx.MX_ERR_OVERLAP  # s_swz inside q
    assert call(a5=1 << 24) == mx.MX_ERR_UNSUPPORTED  # 32-bit offsets within a tile
    assert call(a9=1 << 24) == mx.MX_ERR_UNSUPPORTED
    assert call(a1=0) == mx.MX_OK
    assert call(a2=0, a3=0, a5=0) == mx.MX_OK


def test_quantize_dual_batch_validation():
    L = mx.load()
    f = L.mx_quantize_dual_batch
    J = mx._DualJob
    good = (FAKE, 64, 64, 64, FAKE2, 64, FAKE3, 1, 0x100000000, 64, 0x140000000, 1)
    arr = (J * 3)(J(*good), J(*good), J(*good))
    assert f(ctypes.cast(arr, ctypes.c_void_p), 17, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(ctypes.cast(arr, ctypes.c_void_p), -1, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(None, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(None, 0, STREAM) == mx.MX_OK
    bad = list(good)
    bad[1] = 48                                      # rows % 32 in job 1
    arr[1] = J(*bad)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == mx.MX_ERR_SHAPE
    assert "job 1" in _err(L)
    arr[1] = J(*good)
    other = list(good)
    other[0] = 0x180000000                           # job 2 reads ...
    other[4] = FAKE + 64                             # ... and writes its codes into job 0's input
    arr[2] = J(*other)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == mx.MX_ERR_OVERLAP
    assert "job 0" in _err(L) or "job 2" in _err(L)
    empty = list(good)
    empty[1] = 0
    arr[0] = arr[1] = arr[2] = J(*empty)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == mx.MX_OK


def test_swizzle_validation():
    L = mx.load()
    f = L.mx_scale_swizzle
    assert f(FAKE, 64, 8, 4, FAKE2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 64, 8, 8, FAKE2 + 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 64, 8, 8, FAKE + 16, STREAM) == mx.MX_ERR_OVERLAP
    assert f(0, 64, 8, 8, FAKE2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 0, 8, 8, FAKE2, STREAM) == mx.MX_OK


def test_gemm_validation():
    L = mx.load()
    g = L.mx_gemm
    ok_args = dict(M=64, N=64, K=256, a=FAKE, lda=256, sa=FAKE2, b=FAKE3, ldb=256, sb=FAKE4,
                   c=FAKE4 + (1 << 20), ldc=64, dt=mx.MX_BF16, ws=0, wsb=0)

    def call(**kw):
        a = dict(ok_args, **kw)
        return g(a["M"], a["N"], a["K"], a["a"], a["lda"], a["sa"], a["b"], a["ldb"], a["sb"],
                 a["c"], a["ldc"], a["dt"], a["ws"], a["wsb"], STREAM)

    assert call(K=96) == mx.MX_ERR_UNSUPPORTED
    assert call(K=100, lda=112, ldb=112) == mx.MX_ERR_SHAPE
    assert call(K=0) == mx.MX_ERR_SHAPE
    assert call(dt=7) == mx.MX_ERR_INVALID_ARG
    assert call(M=-1) == mx.MX_ERR_INVALID_ARG
    assert call(lda=128) == mx.MX_ERR_INVALID_ARG
    assert call(ldc=32) == mx.MX_ERR_INVALID_ARG
    assert call(a=FAKE + 8) == mx.MX_ERR_ALIGN
    assert call(lda=264) == mx.MX_ERR_ALIGN
    assert call(sa=FAKE2 + 2) == mx.MX_ERR_ALIGN
    assert call(c=FAKE4 + (1 << 20) + 1) == mx.MX_ERR_ALIGN
    assert call(sb=0) == mx.MX_ERR_INVALID_ARG
    assert call(c=FAKE + 128) == mx.MX_ERR_OVERLAP
    assert call(M=0) == mx.MX_OK
    assert call(N=0) == mx.MX_OK
    assert call(wsb=-1) == mx.MX_ERR_INVALID_ARG


WS = 1 << 36  # fake 256-byte aligned workspace address, far from the operands


def test_gemm_workspace():
    """The split tail's scratch comes from the caller: sized by a host-only
    query, checked for size, alignment and overlap before any launch."""
    L = mx.load()
    q = L.mx_gemm_workspace_bytes
    # 4608 x 4096: 18 x 16 = 288 tiles on 256 compute units (the count this
    # build assumes without a device, and MI355X's) leave 32 tiles; K = 4096
    # has 16 256-K groups: S = min(256 / 32, 16, max(2, floor(sqrt(26 * 2 * 16 / 32)))) = 5
    assert q(4608, 4096, 4096, mx.MX_BF16) == 32 * 5 * 256 * 256 * 4
    assert q(4608, 4096, 4096, mx.MX_F32) == 0          # FP32 C is never split
    assert q(4096, 4096, 4096, mx.MX_BF16) == 0         # 256 tiles: whole rounds
    assert q(4608, 4100, 4096, mx.MX_BF16) == 0         # ragged N: not split
    assert q(4608, 4096, 256, mx.MX_BF16) == 0          # one 256-K group: nothing to split
    assert q(0, 4096, 4096, mx.MX_BF16) == 0 and q(64, 64, 100, mx.MX_BF16) == 0
    need = q(4608, 4096, 4096, mx.MX_BF16)
    g = L.mx_gemm
    M, N, K = 4608, 4096, 4096
    args = lambda ws, wsb, c=FAKE4 + (1 << 20): (M, N, K, FAKE, K, FAKE2, FAKE3, K, FAKE4, c, N, mx.MX_BF16,
                                                ws, wsb, STREAM)
    assert g(*args(0, 0)) == mx.MX_ERR_INVALID_ARG
    assert f"needs a workspace of {need} bytes" in _err(L)
    assert g(*args(WS, need - 1)) == mx.MX_ERR_INVALID_ARG
    assert g(*args(WS + 8, need)) == mx.MX_ERR_ALIGN
    # the workspace over C, and over A's codes
    assert g(*args(FAKE4 + (2 << 20), need)) == mx.MX_ERR_OVERLAP
    assert g(*args(FAKE + 4096, need)) == mx.MX_ERR_OVERLAP


def test_grouped_gemm_validation():
    L = mx.load()
    f = L.mx_grouped_gemm
    base = (4, 100, 64, 256, FAKE4 + (1 << 22), FAKE, 256, FAKE2, FAKE3, FAKE4,
            FAKE4 + (1 << 20), 64, mx.MX_BF16, STREAM)
    assert f(*base[:0], 0, *base[1:]) == mx.MX_ERR_INVALID_ARG
    assert f(*base[:4], 0, *base[5:]) == mx.MX_ERR_INVALID_ARG  # null offsets
    assert f(*base[:4], FAKE4 + (1 << 22) + 4, *base[5:]) == mx.MX_ERR_ALIGN
    assert f(*base[:3], 96, *base[4:]) == mx.MX_ERR_UNSUPPORTED
    # the per-expert tile table holds 1024 experts
    assert f(1025, *base[1:]) == mx.MX_ERR_UNSUPPORTED
    assert "1025 > 1024" in _err(L)
    # C on top of the offsets array
    assert f(*base[:10], FAKE4 + (1 << 22) - 64, *base[11:]) == mx.MX_ERR_OVERLAP
    assert f(*base[:1], 0, *base[2:]) == mx.MX_OK
    # tile numbers are 32-bit: 2^28 rows x 2^21 columns is 2^33 tiles
    assert f(4, 1 << 28, 1 << 21, 256, *base[4:11], 1 << 21, *base[12:]) == mx.MX_ERR_UNSUPPORTED
    assert "2^31" in _err(L)


def test_python_binding_fails_loudly_without_device_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mx.mx_quantize_rowwise(x, q=torch.zeros(4, 64, dtype=torch.uint8),
                               s=torch.zeros(4, 2, dtype=torch.uint8), stream=0)


def test_grouped_k_capacity():
    L = mx.load()
    assert L.mx_grouped_k_capacity(163840, 128) == 163840 + 256 * 128
    assert L.mx_grouped_k_capacity(1, 1) == 512
    assert L.mx_grouped_k_capacity(0, 3) == 768
    assert L.mx_grouped_k_capacity(-1, 3) == 0 and L.mx_grouped_k_capacity(5, 0) == 0


def test_quantize_colwise_grouped_validation():
    L = mx.load()
    f = L.mx_quantize_colwise_grouped
    cap = L.mx_grouped_k_capacity(1000, 4)           # 1024 + 1024
    # x, offsets, pad, qt, st_swz
    args = lambda **kw: [kw.get("x", FAKE), kw.get("rows", 1000), kw.get("cols", 64),
                         kw.get("ld_x", 64), kw.get("off", FAKE2), kw.get("G", 4),
                         kw.get("pad", FAKE2 + 4096), kw.get("qt", FAKE3), kw.get("ld_qt", cap),
                         kw.get("k_cap", cap), kw.get("st", FAKE4), STREAM]
    assert f(*args(cols=48)) == mx.MX_ERR_SHAPE
    assert f(*args(G=0)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(G=1025)) == mx.MX_ERR_UNSUPPORTED
    assert f(*args(k_cap=cap - 256, ld_qt=cap)) == mx.MX_ERR_INVALID_ARG
    assert "mx_grouped_k_capacity" in _err(L)
    assert f(*args(k_cap=cap + 32, ld_qt=cap + 32)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(ld_qt=cap - 16)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(ld_x=32)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(pad=0)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(x=FAKE + 2)) == mx.MX_ERR_ALIGN
    assert f(*args(ld_qt=cap + 8)) == mx.MX_ERR_ALIGN
    assert f(*args(pad=FAKE2 + 4100)) == mx.MX_ERR_ALIGN
    # the padded offsets written over the group offsets; scales inside the codes
    assert f(*args(pad=FAKE2 + 8)) == mx.MX_ERR_OVERLAP
    assert f(*args(st=FAKE3 + 64)) == mx.MX_ERR_OVERLAP
    # 32-bit offsets within a 256-row tile
    assert f(*args(ld_x=1 << 22)) == mx.MX_ERR_UNSUPPORTED
    assert f(*args(ld_qt=1 << 24)) == mx.MX_ERR_UNSUPPORTED


def test_grouped_gemm_wgrad_validation():
    L = mx.load()
    f = L.mx_grouped_gemm_wgrad
    # G, M, N, k_cap, k_offsets, a_q, ld_a, a_s, b_q, ld_b, b_s, c, ld_c, dtype
    args = lambda **kw: [kw.get("G", 4), kw.get("M", 256), kw.get("N", 128), kw.get("K", 2048),
                         kw.get("off", FAKE), kw.get("a", FAKE2), kw.get("ld_a", 2048),
                         kw.get("a_s", FAKE2 + (1 << 24)), kw.get("b", FAKE3),
                         kw.get("ld_b", 2048), kw.get("b_s", FAKE3 + (1 << 24)),
                         kw.get("c", FAKE4), kw.get("ld_c", 128), kw.get("dt", mx.MX_BF16),
                         kw.get("ws", WS), kw.get("wsb", 256), STREAM]
    assert f(*args(G=0)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(G=2000)) == mx.MX_ERR_UNSUPPORTED
    assert f(*args(K=2048 + 128, ld_a=2304, ld_b=2304)) == mx.MX_ERR_SHAPE
    assert "multiple of 256" in _err(L)
    assert f(*args(K=2000)) == mx.MX_ERR_SHAPE
    assert f(*args(off=0)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(off=FAKE + 4)) == mx.MX_ERR_ALIGN
    assert f(*args(ld_c=100)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(dt=7)) == mx.MX_ERR_INVALID_ARG
    # C over A's codes
    assert f(*args(c=FAKE2 + 4096)) == mx.MX_ERR_OVERLAP
    # C (4 experts x 256 rows) reaching the offsets
    assert f(*args(off=FAKE4 + 1000)) == mx.MX_ERR_OVERLAP
    # 2^31 output tiles (1024 experts x 2048 x 1024 tiles): the tile numbers
    # must fit the kernel's 32-bit tile counter
    assert f(*args(G=1024, M=1 << 19, N=1 << 18, ld_c=1 << 18, K=256, ld_a=256, ld_b=256)) == \
        mx.MX_ERR_UNSUPPORTED
    assert "tiles" in _err(L)
    # the tile counter lives in the caller's workspace
    assert L.mx_grouped_gemm_wgrad_workspace_bytes() == 256
    assert f(*args(ws=0, wsb=0)) == mx.MX_ERR_INVALID_ARG
    assert "workspace of 256 bytes" in _err(L)
    assert f(*args(wsb=255)) == mx.MX_ERR_INVALID_ARG
    assert f(*args(ws=WS + 2)) == mx.MX_ERR_ALIGN
    assert f(*args(ws=FAKE4 + 512)) == mx.MX_ERR_OVERLAP       # inside C
    assert f(*args(ws=FAKE + 8)) == mx.MX_ERR_OVERLAP          # over the offsets
    # empty products succeed without a launch
    assert f(*args(M=0)) == mx.MX_OK


def test_moe_dispatch_validation():
    L = mx.load()
    q = L.mx_moe_dispatch_workspace_bytes
    # one int32 count per (256-assignment chunk, expert)
    assert q(20480, 8, 128) == 640 * 128 * 4
    assert q(1, 1, 1) == 4 and q(257, 1, 2) == 2 * 2 * 4
    assert q(0, 8, 128) == 0 and q(10, 8, 2000) == 0
    f = L.mx_moe_dispatch
    T, H, TK, E = 1000, 256, 8, 16
    need = q(T, TK, E)
    # x, tokens, hidden, ld_x, topk_ids, topk, experts, offsets, src, slot, q, ld_q, s_swz, ws, wsb
    base = dict(x=FAKE, T=T, H=H, ldx=H, ids=FAKE2, TK=TK, E=E, off=FAKE2 + (1 << 20),
                src=FAKE2 + (2 << 20), slot=FAKE2 + (3 << 20), q=FAKE3, ldq=H, s=FAKE4, ws=WS, wsb=need)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["x"], a["T"], a["H"], a["ldx"], a["ids"], a["TK"], a["E"], a["off"], a["src"],
                 a["slot"], a["q"], a["ldq"], a["s"], a["ws"], a["wsb"], STREAM)

    assert call(T=-1) == mx.MX_ERR_INVALID_ARG
    assert call(TK=0) == mx.MX_ERR_INVALID_ARG
    assert call(H=100, ldx=112, ldq=112) == mx.MX_ERR_SHAPE
    assert call(H=96, ldx=96, ldq=96) == mx.MX_ERR_UNSUPPORTED
    assert call(E=2000) == mx.MX_ERR_UNSUPPORTED
    assert call(ldq=128) == mx.MX_ERR_INVALID_ARG
    assert call(q=0) == mx.MX_ERR_INVALID_ARG
    assert call(x=FAKE + 8) == mx.MX_ERR_ALIGN
    assert call(off=FAKE2 + (1 << 20) + 4) == mx.MX_ERR_ALIGN
    assert call(src=FAKE3 + 64) == mx.MX_ERR_OVERLAP              # inside q
    # the chunk counts live in the caller's workspace
    assert call(ws=0, wsb=0) == mx.MX_ERR_INVALID_ARG
    assert f"workspace of {need} bytes" in _err(L)
    assert call(wsb=need - 4) == mx.MX_ERR_INVALID_ARG
    assert call(ws=WS + 2) == mx.MX_ERR_ALIGN
    assert call(ws=FAKE3 + 4096) == mx.MX_ERR_OVERLAP            # over q


def test_quantize_dual_experts_validation():
    L = mx.load()
    f = L.mx_quantize_dual_experts
    # x, G, rows, cols, q, s_swz, qt, st_swz
    assert f(FAKE, -1, 64, 64, FAKE2, FAKE3, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 4, 48, 64, FAKE2, FAKE3, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE + 8, 4, 64, 64, FAKE2, FAKE3, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 4, 64, 64, FAKE2, FAKE3 + 2, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_ALIGN
    assert f(0, 4, 64, 64, FAKE2, FAKE3, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_INVALID_ARG
    # the fourth expert's codes (64x64 each) run into s_swz placed 3 experts after q
    assert f(FAKE, 4, 64, 64, FAKE2, FAKE2 + 3 * 4096, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_OVERLAP
    # qt stack over the input stack (4 x 64 x 64 BF16 = 32 KiB)
    assert f(FAKE, 4, 64, 64, FAKE2, FAKE3, FAKE + 30000, FAKE4 + (1 << 20), STREAM) == mx.MX_ERR_OVERLAP
    assert f(FAKE, 0, 64, 64, FAKE2, FAKE3, FAKE4, FAKE4 + (1 << 20), STREAM) == mx.MX_OK


def test_swiglu_quantize_validation():
    L = mx.load()
    f = L.mx_swiglu_quantize
    # gu, rows, F, ld_gu, h, ld_h, q, ld_q, s_swz
    ok_args = [FAKE, 64, 768, 1536, FAKE2, 768, FAKE3, 768, FAKE4]
    a = list(ok_args); a[2] = 48; a[3] = 96
    assert f(*a, STREAM) == mx.MX_ERR_SHAPE
    a = list(ok_args); a[2] = 288; a[3] = 576
    assert f(*a, STREAM) == mx.MX_ERR_UNSUPPORTED
    a = list(ok_args); a[3] = 1000
    assert f(*a, STREAM) == mx.MX_ERR_INVALID_ARG
    a = list(ok_args); a[0] = FAKE + 8
    assert f(*a, STREAM) == mx.MX_ERR_ALIGN
    a = list(ok_args); a[6] = 0
    assert f(*a, STREAM) == mx.MX_ERR_INVALID_ARG
    a = list(ok_args); a[6] = FAKE + 4096      # q inside gu
    assert f(*a, STREAM) == mx.MX_ERR_OVERLAP
    a = list(ok_args); a[1] = 0
    assert f(*a, STREAM) == mx.MX_OK


def test_quantize_rowwise_swz_validation():
    L = mx.load()
    f = L.mx_quantize_rowwise_swz
    # x, rows, cols, ld_x, q, ld_q, s_swz, s_tiles
    assert f(FAKE, 64, 48, 48, FAKE2, 48, FAKE3, 1, STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE, 64, 288, 288, FAKE2, 288, FAKE3, 2, STREAM) == mx.MX_ERR_UNSUPPORTED
    assert f(FAKE, 64, 512, 512, FAKE2, 512, FAKE3, 1, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, -1, 512, 512, FAKE2, 512, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE + 8, 64, 512, 512, FAKE2, 512, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 64, 512, 512, FAKE + 1024, 512, FAKE3, 2, STREAM) == mx.MX_ERR_OVERLAP
    assert f(0, 64, 512, 512, FAKE2, 512, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 0, 512, 512, FAKE2, 512, FAKE3, 2, STREAM) == mx.MX_OK


def test_quantize_rowwise_swz_batch_validation():
    L = mx.load()
    f = L.mx_quantize_rowwise_swz_batch
    J = mx._RowJob
    good = (FAKE, 64, 512, 512, FAKE2, 512, FAKE3, 2)
    arr = (J * 3)(J(*good), J(*good), J(*good))
    assert f(ctypes.cast(arr, ctypes.c_void_p), 9, STREAM) == mx.MX_ERR_INVALID_ARG
    assert "0..8" in _err(L)
    assert f(ctypes.cast(arr, ctypes.c_void_p), -1, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(None, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(None, 0, STREAM) == mx.MX_OK
    for i, v, code in ((2, 48, mx.MX_ERR_SHAPE), (2, 288, mx.MX_ERR_UNSUPPORTED), (7, 1, mx.MX_ERR_INVALID_ARG),
                       (1, -1, mx.MX_ERR_INVALID_ARG), (0, FAKE + 8, mx.MX_ERR_ALIGN),
                       (4, FAKE + 1024, mx.MX_ERR_OVERLAP), (6, 0, mx.MX_ERR_INVALID_ARG)):
        bad = list(good)
        bad[i] = v
        if i == 2:
            bad[3] = bad[5] = v
        arr[1] = J(*bad)
        assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == code, (i, v)
        assert "job 1" in _err(L)
    arr[1] = J(*good)
    other = list(good)
    other[0] = 0x180000000                           # job 2 reads ...
    other[6] = FAKE + 4096                           # ... and writes its scales into job 0's input
    arr[2] = J(*other)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == mx.MX_ERR_OVERLAP
    assert "job 0" in _err(L)
    empty = list(good)
    empty[1] = 0
    arr[0] = arr[1] = arr[2] = J(*empty)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3, STREAM) == mx.MX_OK


def test_quantize_colwise_swz_validation():
    L = mx.load()
    f = L.mx_quantize_colwise_swz
    # x, rows, cols, ld_x, qt, ld_qt, st_swz, st_tiles
    assert f(FAKE, 48, 64, 64, FAKE2, 48, FAKE3, 1, STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE, 256, 60, 64, FAKE2, 256, FAKE3, 1, STREAM) == mx.MX_ERR_SHAPE
    assert f(FAKE, 288, 64, 64, FAKE2, 288, FAKE3, 2, STREAM) == mx.MX_ERR_UNSUPPORTED
    assert f(FAKE, 256, 40, 40, FAKE2, 256, FAKE3, 1, STREAM) == mx.MX_ERR_UNSUPPORTED
    assert f(FAKE, 512, 64, 64, FAKE2, 512, FAKE3, 1, STREAM) == mx.MX_ERR_INVALID_ARG  # st_tiles
    assert f(FAKE, 512, 64, 64, FAKE2, 256, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG  # ld_qt
    assert f(FAKE, -256, 64, 64, FAKE2, 512, FAKE3, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 512, 64, 64, FAKE2 + 8, 512, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 512, 64, 64, FAKE2, 520, FAKE3, 2, STREAM) == mx.MX_ERR_ALIGN
    assert f(FAKE, 512, 64, 64, FAKE + 4096, 512, FAKE3, 2, STREAM) == mx.MX_ERR_OVERLAP
    assert f(FAKE, 512, 64, 64, FAKE2, 512, FAKE2 + 512, 2, STREAM) == mx.MX_ERR_OVERLAP
    assert f(FAKE, 512, 64, 64, FAKE2, 512, 0, 2, STREAM) == mx.MX_ERR_INVALID_ARG
    assert f(FAKE, 0, 64, 64, FAKE2, 0, FAKE3, 0, STREAM) == mx.MX_OK


def test_quantize_dual_grouped_validation():
    L = mx.load()
    f = L.mx_quantize_dual_grouped
    cap = L.mx_grouped_k_capacity(1000, 4)
    # x, rows, cols, ld_x, offsets, G, pad, q, ld_q, s_swz, qt, ld_qt, k_cap, st_swz
    base = dict(x=FAKE, rows=1000, cols=256, ld_x=256, off=FAKE2, G=4, pad=FAKE2 + 4096, q=FAKE3,
                ld_q=256, s=FAKE3 + (1 << 24), qt=FAKE4, ld_qt=cap, k_cap=cap, st=FAKE4 + (1 << 24))
    order = ["x", "rows", "cols", "ld_x", "off", "G", "pad", "q", "ld_q", "s", "qt", "ld_qt", "k_cap", "st"]
    call = lambda **kw: f(*[kw.get(k, base[k]) for k in order], STREAM)
    assert call(cols=288, ld_x=288, ld_q=288) == mx.MX_ERR_UNSUPPORTED
    assert call(cols=48, ld_x=48, ld_q=48) == mx.MX_ERR_SHAPE
    assert call(ld_q=128) == mx.MX_ERR_INVALID_ARG
    assert call(q=0) == mx.MX_ERR_INVALID_ARG
    assert call(q=FAKE3 + 8) == mx.MX_ERR_ALIGN
    assert call(ld_q=264) == mx.MX_ERR_ALIGN
    assert call(s=FAKE3 + (1 << 24) + 2) == mx.MX_ERR_ALIGN
    assert call(s=FAKE3 + 1000) == mx.MX_ERR_OVERLAP        # row-wise scales inside the codes
    assert call(k_cap=cap - 256, ld_qt=cap) == mx.MX_ERR_INVALID_ARG
    assert call(ld_q=1 << 24) == mx.MX_ERR_UNSUPPORTED
    assert call(ld_x=1 << 22) == mx.MX_ERR_UNSUPPORTED


def test_swiglu_quantize_dual_grouped_validation():
    """The fused SwiGLU + row-wise + per-expert column-wise quantization checks
    its arguments like mx_quantize_dual_grouped, with the gate/up input twice
    as wide as the quantized h, before any launch."""
    L = mx.load()
    f = L.mx_swiglu_quantize_dual_grouped
    cap = L.mx_grouped_k_capacity(1000, 4)
    # gu, rows, F, ld_gu, offsets, G, pad, q, ld_q, s_swz, qt, ld_qt, k_cap, st_swz
    base = dict(gu=FAKE, rows=1000, F=256, ld_gu=512, off=FAKE2, G=4, pad=FAKE2 + 4096, q=FAKE3,
                ld_q=256, s=FAKE3 + (1 << 24), qt=FAKE4, ld_qt=cap, k_cap=cap, st=FAKE4 + (1 << 24))
    order = ["gu", "rows", "F", "ld_gu", "off", "G", "pad", "q", "ld_q", "s", "qt", "ld_qt", "k_cap", "st"]
    call = lambda **kw: f(*[kw.get(k, base[k]) for k in order], STREAM)
    assert call(ld_gu=256) == mx.MX_ERR_INVALID_ARG         # the up half does not fit
    assert call(F=288, ld_gu=576, ld_q=288) == mx.MX_ERR_UNSUPPORTED
    assert call(F=48, ld_gu=96, ld_q=48) == mx.MX_ERR_SHAPE
    assert call(F=0) == mx.MX_ERR_INVALID_ARG
    assert call(rows=-1) == mx.MX_ERR_INVALID_ARG
    assert call(G=0) == mx.MX_ERR_INVALID_ARG
    assert call(G=1025) == mx.MX_ERR_UNSUPPORTED
    assert call(ld_q=128) == mx.MX_ERR_INVALID_ARG
    assert call(q=0) == mx.MX_ERR_INVALID_ARG
    assert call(gu=0) == mx.MX_ERR_INVALID_ARG
    assert call(gu=FAKE + 8) == mx.MX_ERR_ALIGN
    assert call(ld_gu=516) == mx.MX_ERR_ALIGN
    assert call(q=FAKE3 + 8) == mx.MX_ERR_ALIGN
    assert call(s=FAKE3 + (1 << 24) + 2) == mx.MX_ERR_ALIGN
    assert call(s=FAKE3 + 1000) == mx.MX_ERR_OVERLAP        # row-wise scales inside the codes
    assert call(q=FAKE + 4096) == mx.MX_ERR_OVERLAP         # codes inside the input
    assert call(k_cap=cap - 256, ld_qt=cap) == mx.MX_ERR_INVALID_ARG
    assert call(ld_q=1 << 24) == mx.MX_ERR_UNSUPPORTED
    assert call(ld_gu=1 << 22) == mx.MX_ERR_UNSUPPORTED
    assert "ld_gu" in mx.mx_last_error()


def test_moe_dispatch_dual_grouped_validation():
    """The dispatch that also writes the per-expert column-wise operand checks
    mx_moe_dispatch's arguments and the grouped operand's (capacity, alignment,
    overlap, the 32-bit offset bounds) before any launch."""
    L = mx.load()
    f = L.mx_moe_dispatch_dual_grouped
    T, H, TK, E = 1000, 256, 8, 16
    need = L.mx_moe_dispatch_workspace_bytes(T, TK, E)
    cap = L.mx_grouped_k_capacity(T * TK, E)
    # x, tokens, hidden, ld_x, topk_ids, topk, experts, offsets, src, slot, q, ld_q, s_swz,
    # pad, qt, ld_qt, k_cap, st_swz, ws, wsb
    base = dict(x=FAKE, T=T, H=H, ldx=H, ids=FAKE2, TK=TK, E=E, off=FAKE2 + (1 << 20),
                src=FAKE2 + (2 << 20), slot=FAKE2 + (3 << 20), q=FAKE3, ldq=H, s=FAKE4,
                pad=FAKE2 + (4 << 20), qt=FAKE3 + (64 << 20), ldqt=cap, kcap=cap, st=FAKE4 + (64 << 20),
                ws=WS, wsb=need)
    order = ["x", "T", "H", "ldx", "ids", "TK", "E", "off", "src", "slot", "q", "ldq", "s", "pad", "qt", "ldqt",
             "kcap", "st", "ws", "wsb"]

    def call(**kw):
        a = dict(base, **kw)
        return f(*[a[k] for k in order], STREAM)

    assert call(T=-1) == mx.MX_ERR_INVALID_ARG
    assert call(H=96, ldx=96, ldq=96) == mx.MX_ERR_UNSUPPORTED
    assert call(E=2000) == mx.MX_ERR_UNSUPPORTED
    assert call(q=0) == mx.MX_ERR_INVALID_ARG
    assert call(kcap=cap - 256, ldqt=cap) == mx.MX_ERR_INVALID_ARG
    assert call(kcap=cap + 128, ldqt=cap + 128) == mx.MX_ERR_INVALID_ARG
    assert call(ldqt=cap - 16) == mx.MX_ERR_INVALID_ARG
    assert call(qt=0) == mx.MX_ERR_INVALID_ARG
    assert call(pad=0) == mx.MX_ERR_INVALID_ARG
    assert call(qt=FAKE3 + (64 << 20) + 8) == mx.MX_ERR_ALIGN
    assert call(ldqt=cap + 8) == mx.MX_ERR_ALIGN
    assert call(st=FAKE4 + (64 << 20) + 2) == mx.MX_ERR_ALIGN
    assert call(pad=FAKE2 + (4 << 20) + 4) == mx.MX_ERR_ALIGN
    assert call(qt=FAKE3) == mx.MX_ERR_OVERLAP                    # column-wise codes over q
    assert call(pad=FAKE2 + (1 << 20)) == mx.MX_ERR_OVERLAP       # pad over offsets
    assert call(ws=FAKE3 + (64 << 20)) == mx.MX_ERR_OVERLAP       # workspace over qt
    far = 1 << 40  # a fake x far from the other buffers, so only the size rules apply
    assert call(x=far, ldx=1 << 22) == mx.MX_ERR_UNSUPPORTED
    assert call(x=far, ldx=1 << 21) == mx.MX_ERR_UNSUPPORTED   # x of 4 GiB: past 32-bit offsets
    assert "x below 2^31" in mx.mx_last_error()


def test_moe_dispatch_noalloc_validation():
    """The variant without a workspace checks its arguments like
    mx_moe_dispatch and refuses routings whose chunk counts would not fit its
    4 MiB device array, before any launch."""
    L = mx.load()
    f = L.mx_moe_dispatch_noalloc
    H, TK = 256, 8

    def call(T, E, **kw):
        a = dict(x=FAKE, ids=FAKE2, off=FAKE2 + (64 << 20), src=FAKE2 + (128 << 20),
                 slot=FAKE2 + (192 << 20), q=FAKE3, s=FAKE4)
        a.update(kw)
        return f(a["x"], T, H, H, a["ids"], TK, E, a["off"], a["src"], a["slot"], a["q"], H, a["s"], STREAM)

    # 262 144 assignments over 1024 experts: 1024 chunks x 1024 x 4 bytes = 4 MiB
    assert L.mx_moe_dispatch_workspace_bytes(32768, TK, 1024) == 4 << 20
    # one chunk more does not fit
    assert L.mx_moe_dispatch_workspace_bytes(32800, TK, 1024) > 4 << 20
    assert call(32800, 1024) == mx.MX_ERR_UNSUPPORTED
    assert "4194304" in _err(L) and "mx_moe_dispatch" in _err(L)
    assert call(300000, 128) == mx.MX_ERR_UNSUPPORTED
    # the same argument checks as mx_moe_dispatch
    assert call(-1, 16) == mx.MX_ERR_INVALID_ARG
    assert call(100, 2000) == mx.MX_ERR_UNSUPPORTED
    assert call(100, 16, q=0) == mx.MX_ERR_INVALID_ARG
    assert call(100, 16, x=FAKE + 8) == mx.MX_ERR_ALIGN
    assert call(100, 16, src=FAKE3 + 64) == mx.MX_ERR_OVERLAP
