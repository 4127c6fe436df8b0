"""CPU oracle for MXFP8 quantization, scale rearrangement and block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library in
``mxfp8_block_scaled_08_amd`` never does and shares no code with it.

The quantization, rearrangement, GEMM, per-expert column-wise and SwiGLU
arithmetic lives in ``oracle/mx_oracle.c`` (plain scalar C, double
precision); for those this module only marshals numpy arrays into it.  Two
definitions are written here in plain numpy instead, because they are index
work and one weighted sum rather than number formats: ``moe_dispatch`` (the
stable sort of routed assignments by expert) and ``moe_combine`` (the
weighted sum of each token's expert outputs, in double precision), plus the
grouped padding offsets and capacity (integer arithmetic).  The sources
followed are named in the header of the C file and beside each function: the
MXFP8 RL paper "End-to-End MXFP8 Reinforcement Learning on Blackwell"
(Figure 1, Table 2, Table 6, Table 10) for what the path computes, and the
OCP MX v1.0 shared-scale rule for the bytes.  ``mx_oracle_ref.py`` is a
second, independent implementation of the quantization, rearrangement and
GEMM (numpy, different rounding route) that tests/test_oracle_agreement.py
checks against this one.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    """Load (building on first use if absent) the oracle's shared library."""
    global _lib
    if _lib is None:
        path = LIB
        if not os.path.exists(path):
            path = build_oracle()
        L = ctypes.CDLL(path)
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_scale_code.restype = ctypes.c_uint8
        L.oracle_scale_code.argtypes = [ctypes.c_double]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_swizzled_bytes.restype = _i64
        L.oracle_swizzled_bytes.argtypes = [_i64, _i64]
        L.oracle_swizzle_offset.restype = _i64
        L.oracle_swizzle_offset.argtypes = [_i64, _i64, _i64]
        L.oracle_dequant.restype = ctypes.c_double
        L.oracle_dequant.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
        L.oracle_e4m3_encode_array.argtypes = [_f64p, _i64, _u8p]
        L.oracle_e4m3_decode_array.argtypes = [_u8p, _i64, _f64p]
        L.oracle_scale_code_array.argtypes = [_f64p, _i64, _u8p]
        L.oracle_quantize_rowwise.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _u8p, _i64]
        L.oracle_quantize_colwise.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _u8p, _i64]
        L.oracle_scale_swizzle.argtypes = [_u8p, _i64, _i64, _i64, _u8p]
        L.oracle_scale_unswizzle.argtypes = [_u8p, _i64, _i64, _u8p, _i64]
        L.oracle_dequantize_rowwise.argtypes = [_u8p, _i64, _i64, _i64, _u8p, _i64, _f64p]
        L.oracle_gemm.argtypes = [_i64, _i64, _i64, _u8p, _i64, _u8p, _i64, _u8p, _i64, _u8p,
                                  _i64, _f64p, _f64p]
        L.oracle_gemm_sampled.argtypes = [_i64, _i64p, _i64p, _i64, _u8p, _i64, _u8p, _i64,
                                          _u8p, _i64, _u8p, _i64, _f64p, _f64p]
        L.oracle_grouped_gemm_sampled.argtypes = [_i64, _i64p, _i64p, _i64, _i64p, _i64, _i64,
                                                  _u8p, _i64, _u8p, _i64, _u8p, _i64, _u8p,
                                                  _i64, _f64p, _f64p]
        L.oracle_grouped_pad_offsets.argtypes = [_i64, _i64p, _i64p]
        L.oracle_swiglu_f64.restype = ctypes.c_double
        L.oracle_swiglu_f64.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_swiglu_bf16.argtypes = [_u16p, _i64, _i64, _i64, _u16p]
        L.oracle_quantize_colwise_grouped.argtypes = [_u16p, _i64, _i64, _i64, _i64p, _i64p,
                                                      _u8p, _i64, _u8p, _i64]
        L.oracle_grouped_wgrad_sampled.argtypes = [_i64, _i64p, _i64p, _i64p, _i64p, _u8p, _i64,
                                                   _u8p, _i64, _u8p, _i64, _u8p, _i64, _f64p,
                                                   _f64p]
        _lib = L
    return _lib


def _p(a, typ):
    return a.ctypes.data_as(typ)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---- scalars -------------------------------------------------------------

def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e4m3_encode(t: float) -> int:
    return lib().oracle_e4m3_encode(t)


def scale_code(amax: float) -> int:
    return lib().oracle_scale_code(amax)


def e8m0_decode(code: int) -> float:
    return lib().oracle_e8m0_decode(code)


def dequant(q: int, c: int) -> float:
    return lib().oracle_dequant(q, c)


# ---- arrays ----------------------------------------------------------------

def e4m3_encode_array(t) -> np.ndarray:
    t = _c(t, np.float64)
    out = np.empty(t.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(t, _f64p), t.size, _p(out, _u8p))
    return out


def e4m3_decode_array(q) -> np.ndarray:
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().oracle_e4m3_decode_array(_p(q, _u8p), q.size, _p(out, _f64p))
    return out


def scale_code_array(amax) -> np.ndarray:
    a = _c(amax, np.float64)
    out = np.empty(a.shape, np.uint8)
    lib().oracle_scale_code_array(_p(a, _f64p), a.size, _p(out, _u8p))
    return out


def quantize_rowwise(x_bits):
    """x_bits: uint16 [rows, cols] of BF16 bit patterns -> (q [rows, cols], s [rows, cols/32])."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    assert cols % 32 == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    lib().oracle_quantize_rowwise(_p(x, _u16p), rows, cols, cols, _p(q, _u8p), cols,
                                  _p(s, _u8p), cols // 32)
    return q, s


def quantize_colwise(x_bits):
    """x_bits: uint16 [rows, cols] -> (qt [cols, rows], st [cols, rows/32])."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    assert rows % 32 == 0
    qt = np.empty((cols, rows), np.uint8)
    st = np.empty((cols, rows // 32), np.uint8)
    lib().oracle_quantize_colwise(_p(x, _u16p), rows, cols, cols, _p(qt, _u8p), rows,
                                  _p(st, _u8p), rows // 32)
    return qt, st


def swizzled_bytes(rows: int, kblocks: int) -> int:
    return lib().oracle_swizzled_bytes(rows, kblocks)


def swizzle_offset(row: int, blk: int, kblocks: int) -> int:
    return lib().oracle_swizzle_offset(row, blk, kblocks)


def scale_swizzle(s) -> np.ndarray:
    s = _c(s, np.uint8)
    rows, kb = s.shape
    out = np.empty(swizzled_bytes(rows, kb), np.uint8)
    lib().oracle_scale_swizzle(_p(s, _u8p), rows, kb, kb, _p(out, _u8p))
    return out


def scale_unswizzle(buf, rows: int, kblocks: int) -> np.ndarray:
    buf = _c(buf, np.uint8)
    assert buf.size >= swizzled_bytes(rows, kblocks)
    s = np.empty((rows, kblocks), np.uint8)
    lib().oracle_scale_unswizzle(_p(buf, _u8p), rows, kblocks, _p(s, _u8p), kblocks)
    return s


def dequantize_rowwise(q, s) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float64)
    lib().oracle_dequantize_rowwise(_p(q, _u8p), rows, cols, cols, _p(s, _u8p), s.shape[1],
                                    _p(out, _f64p))
    return out


def gemm(qa, sa, qb, sb):
    """C = deq(A) deq(B)^T and Bnd = |deq(A)| |deq(B)|^T, both float64 [M, N].

    qa [M, K], sa [M, K/32], qb [N, K], sb [N, K/32], plain (unrearranged) scales."""
    qa, sa, qb, sb = (_c(a, np.uint8) for a in (qa, sa, qb, sb))
    M, K = qa.shape
    N = qb.shape[0]
    assert qb.shape[1] == K and sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    c = np.empty((M, N), np.float64)
    bnd = np.empty((M, N), np.float64)
    lib().oracle_gemm(M, N, K, _p(qa, _u8p), K, _p(sa, _u8p), K // 32, _p(qb, _u8p), K,
                      _p(sb, _u8p), K // 32, _p(c, _f64p), _p(bnd, _f64p))
    return c, bnd


def gemm_sampled(rows, cols, qa, sa, qb, sb):
    """Entries (rows[e], cols[e]) of deq(A) deq(B)^T, with their bounds."""
    qa, sa, qb, sb = (_c(a, np.uint8) for a in (qa, sa, qb, sb))
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    K = qa.shape[1]
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < qa.shape[0])
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < qb.shape[0])
    c = np.empty(rows.size, np.float64)
    bnd = np.empty(rows.size, np.float64)
    lib().oracle_gemm_sampled(rows.size, _p(rows, _i64p), _p(cols, _i64p), K, _p(qa, _u8p), K,
                              _p(sa, _u8p), K // 32, _p(qb, _u8p), K, _p(sb, _u8p), K // 32,
                              _p(c, _f64p), _p(bnd, _f64p))
    return c, bnd


def grouped_gemm_sampled(rows, cols, offsets, qa, sa, qb, sb):
    """Per-expert product: row i in [offsets[g], offsets[g+1]) uses expert g.

    qa [M_total, K], sa [M_total, K/32], qb [G, N, K], sb [G, N, K/32]."""
    qa, sa, qb, sb = (_c(a, np.uint8) for a in (qa, sa, qb, sb))
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    offsets = _c(offsets, np.int64)
    G, N, K = qb.shape
    assert offsets.size == G + 1 and offsets[0] == 0 and offsets[-1] == qa.shape[0]
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < qa.shape[0])
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < N)
    c = np.empty(rows.size, np.float64)
    bnd = np.empty(rows.size, np.float64)
    lib().oracle_grouped_gemm_sampled(rows.size, _p(rows, _i64p), _p(cols, _i64p), G,
                                      _p(offsets, _i64p), N, K, _p(qa, _u8p), K, _p(sa, _u8p),
                                      K // 32, _p(qb, _u8p), K, _p(sb, _u8p), K // 32,
                                      _p(c, _f64p), _p(bnd, _f64p))
    return c, bnd


def grouped_gemm(offsets, qa, sa, qb, sb):
    """Full per-expert product (small sizes): float64 [M_total, N] and its bound."""
    G, N, K = np.asarray(qb).shape
    M = np.asarray(qa).shape[0]
    rows = np.repeat(np.arange(M, dtype=np.int64), N)
    cols = np.tile(np.arange(N, dtype=np.int64), M)
    c, bnd = grouped_gemm_sampled(rows, cols, offsets, qa, sa, qb, sb)
    return c.reshape(M, N), bnd.reshape(M, N)


def moe_dispatch(topk_ids, num_experts: int):
    """Rows sorted by expert, stably: the MoE layer's expert GEMMs run per expert
    on rows sorted by expert ("End-to-End MXFP8 Reinforcement Learning on
    Blackwell", Table 2: 128 experts, 8 routed per token).  Assignment
    a = t*topk + j sends token t to expert e = topk_ids[t][j]; ids outside
    [0, num_experts) are not routed.  Assignment a lands on row offsets[e] +
    (number of assignments a' < a to the same expert).

    Returns (offsets int64 [G+1], src_token int32 [n]: token of each row, -1
    past the routed count, slot int32 [n]: row of each assignment, -1 if not
    routed); n = tokens * topk."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    e = ids.reshape(-1)
    n = e.size
    valid = (e >= 0) & (e < num_experts)
    offsets = np.zeros(num_experts + 1, np.int64)
    offsets[1:] = np.cumsum(np.bincount(e[valid], minlength=num_experts))
    # a stable sort by expert (library sort as one step); unrouted ones last
    order = np.argsort(np.where(valid, e, num_experts), kind="stable")
    routed = int(valid.sum())
    slot = np.full(n, -1, np.int32)
    slot[order[:routed]] = np.arange(routed, dtype=np.int32)
    src = np.full(n, -1, np.int32)
    src[:routed] = (order[:routed] // topk).astype(np.int32)
    return offsets, src, slot


def moe_combine(y_bits, slot, weights):
    """out[t] = sum_j weights[t][j] * y[slot[t*topk + j]] in float64, skipping
    slots outside [0, rows of y); y given as BF16 bit patterns [n][hidden]."""
    y = np.asarray(y_bits, np.uint16).astype(np.uint32) << 16
    y = y.view(np.float32).astype(np.float64)
    w = np.asarray(weights, np.float32).astype(np.float64)
    tokens, topk = w.shape
    slot = np.asarray(slot, np.int64).reshape(tokens, topk)
    out = np.zeros((tokens, y.shape[1]), np.float64)
    bnd = np.zeros_like(out)
    for j in range(topk):
        p = slot[:, j]
        ok = (p >= 0) & (p < y.shape[0])
        rows = y[np.where(ok, p, 0)]
        term = np.where(ok[:, None], w[:, j:j + 1] * rows, 0.0)
        out += term
        bnd += np.abs(term)
    return out, bnd


# ---- MoE backward ----------------------------------------------------------
# The expert weight gradient dW_g = dY_g^T X_g of the update_actor stage
# ("End-to-End MXFP8 Reinforcement Learning on Blackwell", Table 8; Table 2
# for the 128-expert top-8 model) contracts over the expert's own token rows,
# with both operands quantized column-wise in 32-row blocks that never hold
# rows of two experts.  Layout: expert g's rows become columns
# [pad[g], pad[g+1]) of the transposed operand, each range max(256, m_g
# rounded up to 256) long, the rows past m_g taken as zeros.


def grouped_pad_offsets(offsets) -> np.ndarray:
    """pad int64 [G+1]: pad[0] = 0, pad[g+1] = pad[g] + max(256, ceil(m_g/256)*256)."""
    offsets = _c(offsets, np.int64)
    G = offsets.size - 1
    pad = np.empty(G + 1, np.int64)
    lib().oracle_grouped_pad_offsets(G, _p(offsets, _i64p), _p(pad, _i64p))
    return pad


def grouped_k_capacity(rows_total: int, G: int) -> int:
    """A column count that holds pad[G] for any split of rows_total rows into G
    experts: each range exceeds its m_g by at most 256."""
    return (rows_total + 255) // 256 * 256 + 256 * G


def quantize_colwise_grouped(x_bits, offsets, k_cap: int):
    """x_bits uint16 [rows_total, cols], rows sorted by expert ->
    (qt uint8 [cols, k_cap], st uint8 [cols, k_cap/32], pad int64 [G+1]).
    Expert g's column-wise blocks of its own rows land in columns
    [pad[g], pad[g+1]); columns past pad[G] are zero here (the library
    leaves them unwritten)."""
    x = _c(x_bits, np.uint16)
    offsets = _c(offsets, np.int64)
    rows, cols = x.shape
    G = offsets.size - 1
    assert offsets[0] == 0 and offsets[-1] == rows and (np.diff(offsets) >= 0).all()
    pad = grouped_pad_offsets(offsets)
    assert k_cap % 256 == 0 and pad[-1] <= k_cap
    qt = np.zeros((cols, k_cap), np.uint8)
    st = np.zeros((cols, k_cap // 32), np.uint8)
    if rows == 0:
        x = np.zeros((1, cols), np.uint16)  # a valid pointer; no row is read
    lib().oracle_quantize_colwise_grouped(_p(x, _u16p), cols, cols, G, _p(offsets, _i64p),
                                          _p(pad, _i64p), _p(qt, _u8p), k_cap, _p(st, _u8p),
                                          k_cap // 32)
    return qt, st, pad


def grouped_wgrad_sampled(groups, rows, cols, pad, qa, sa, qb, sb):
    """Entries C_g[rows[e]][cols[e]] (g = groups[e]) of the per-expert product
    C_g = deq(A)[:, pad[g]:pad[g+1]] deq(B)[:, pad[g]:pad[g+1]]^T, with bounds.
    qa [M, Kc], sa [M, Kc/32], qb [N, Kc], sb [N, Kc/32]."""
    qa, sa, qb, sb = (_c(a, np.uint8) for a in (qa, sa, qb, sb))
    groups, rows, cols, pad = (_c(a, np.int64) for a in (groups, rows, cols, pad))
    Kc = qa.shape[1]
    assert qb.shape[1] == Kc and sa.shape[1] == Kc // 32 and sb.shape[1] == Kc // 32
    assert groups.shape == rows.shape == cols.shape
    assert pad[-1] <= Kc and (pad % 32 == 0).all()
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < qa.shape[0])
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < qb.shape[0])
    assert groups.size == 0 or (groups.min() >= 0 and groups.max() < pad.size - 1)
    c = np.empty(rows.size, np.float64)
    bnd = np.empty(rows.size, np.float64)
    lib().oracle_grouped_wgrad_sampled(rows.size, _p(groups, _i64p), _p(rows, _i64p),
                                       _p(cols, _i64p), _p(pad, _i64p), _p(qa, _u8p), Kc,
                                       _p(sa, _u8p), Kc // 32, _p(qb, _u8p), Kc, _p(sb, _u8p),
                                       Kc // 32, _p(c, _f64p), _p(bnd, _f64p))
    return c, bnd


def grouped_wgrad(pad, qa, sa, qb, sb):
    """Every entry (small sizes): float64 [G, M, N] and its bound."""
    pad = _c(pad, np.int64)
    G = pad.size - 1
    M, N = np.asarray(qa).shape[0], np.asarray(qb).shape[0]
    g, i, j = np.meshgrid(np.arange(G), np.arange(M), np.arange(N), indexing="ij")
    c, bnd = grouped_wgrad_sampled(g.ravel(), i.ravel(), j.ravel(), pad, qa, sa, qb, sb)
    return c.reshape(G, M, N), bnd.reshape(G, M, N)


# ---- SwiGLU between the MoE expert projections --------------------------
# Qwen3's expert MLP ("End-to-End MXFP8 Reinforcement Learning on Blackwell",
# Table 2: Qwen3-30B-A3B) feeds the down projection with h = silu(g) * u,
# silu(g) = g / (1 + exp(-g)); g and u are the gate and up halves of the
# gate_up product.  Activations are BF16 (Figure 1), so h is rounded once to
# BF16 and then quantized row-wise as the down projection's A operand.


def swiglu_f64(g: float, u: float) -> float:
    return lib().oracle_swiglu_f64(g, u)


def double_to_bf16(v: float) -> int:
    """Nearest BF16 bit pattern (ties to even), one rounding from double."""
    return lib().oracle_double_to_bf16(v)


def swiglu_bf16(gu_bits):
    """gu_bits uint16 [rows, 2F] (gate | up) -> h uint16 [rows, F] (BF16 bits)."""
    gu = _c(gu_bits, np.uint16)
    rows, F2 = gu.shape
    assert F2 % 2 == 0
    F = F2 // 2
    h = np.empty((rows, F), np.uint16)
    if rows:
        lib().oracle_swiglu_bf16(_p(gu, _u16p), rows, F, F2, _p(h, _u16p))
    return h


def swiglu_quantize(gu_bits):
    """SwiGLU then row-wise MXFP8: (h [rows, F] BF16 bits, q [rows, F], s [rows, F/32])."""
    h = swiglu_bf16(gu_bits)
    q, s = quantize_rowwise(h)
    return h, q, s
