"""MI355X (gfx950) MXFP8 hot path: quantize, scale rearrangement, block-scaled GEMM.

A thin Python binding over the C ABI of ``libmxfp8.so`` (declared in
``include/mxfp8.h``).  Every function here only marshals torch tensors into
pointers, sizes and the current HIP stream; all computation runs in the
library's HIP kernels.  If the shared library is missing, ``load()`` raises:
there is no fallback path.

The operations are those of the MXFP8 learner/sampler hot path in
"End-to-End MXFP8 Reinforcement Learning on Blackwell" (Figure 1: quantize
the weights with the learner's quantizer, MXFP8 GEMMs; Table 6: GEMM,
quantization and scale-rearrangement kernels; Table 2: dense Qwen3-8B and
the 128-expert Qwen3-30B-A3B MoE).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MxError", "load", "lib_path", "mx_abi_version", "mx_status_string", "mx_last_error", "mx_quantize_rowwise",
    "mx_quantize_colwise", "mx_scale_swizzled_bytes", "mx_scale_swizzle", "mx_gemm",
    "mx_grouped_gemm", "mx_quantize_dual", "mx_quantize_dual_batch", "mx_quantize_dual_experts",
    "mx_moe_dispatch", "mx_moe_dispatch_dual_grouped", "mx_moe_combine", "mx_grouped_k_capacity", "mx_quantize_colwise_grouped",
    "mx_grouped_gemm_wgrad", "mx_swiglu_quantize", "mx_quantize_rowwise_swz",
    "mx_quantize_rowwise_swz_batch", "mx_quantize_colwise_swz",
    "mx_quantize_dual_grouped", "mx_swiglu_quantize_dual_grouped", "mx_gemm_workspace_bytes", "mx_moe_dispatch_workspace_bytes",
    "mx_grouped_gemm_wgrad_workspace_bytes", "mx_moe_dispatch_noalloc", "MX_OK", "MX_ERR_INVALID_ARG", "MX_ERR_SHAPE", "MX_ERR_ALIGN",
    "MX_ERR_OVERLAP", "MX_ERR_UNSUPPORTED", "MX_ERR_HIP", "MX_BF16", "MX_F32",
]

MX_OK, MX_ERR_INVALID_ARG, MX_ERR_SHAPE, MX_ERR_ALIGN = 0, 1, 2, 3
MX_ERR_OVERLAP, MX_ERR_UNSUPPORTED, MX_ERR_HIP = 4, 5, 6
MX_BF16, MX_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8.so")
_lib: Optional[ctypes.CDLL] = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class MxError(RuntimeError):
    """A non-MX_OK status from the library, with its message."""

    def __init__(self, fn: str, status: int, msg: str):
        self.status = status
        super().__init__(f"{fn} -> {_status_name(status)}: {msg}")


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libmxfp8.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} not found: build it first (python -c 'import __graft_entry__ as g; "
            "g.build()'); there is no CPU fallback")
    L = ctypes.CDLL(_LIB_PATH)
    L.mx_abi_version.restype = ctypes.c_int
    L.mx_abi_version.argtypes = []
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_status_string.argtypes = [ctypes.c_int]
    L.mx_last_error.restype = ctypes.c_char_p
    L.mx_last_error.argtypes = []
    L.mx_scale_swizzled_bytes.restype = _i64
    L.mx_scale_swizzled_bytes.argtypes = [_i64, _i64]
    for name in ("mx_quantize_rowwise", "mx_quantize_colwise"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
    L.mx_scale_swizzle.restype = ctypes.c_int
    L.mx_scale_swizzle.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp]
    L.mx_quantize_dual.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                   _i64, _vp]
    L.mx_quantize_dual.restype = ctypes.c_int
    L.mx_quantize_dual_batch.argtypes = [ctypes.c_void_p, ctypes.c_int, _vp]
    L.mx_quantize_dual_batch.restype = ctypes.c_int
    L.mx_moe_dispatch.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64,
                                  _vp, _vp, _i64, _vp]
    L.mx_moe_dispatch_noalloc.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                          _i64, _vp, _vp]
    L.mx_moe_dispatch_noalloc.restype = ctypes.c_int
    L.mx_moe_dispatch_workspace_bytes.restype = _i64
    L.mx_moe_dispatch_workspace_bytes.argtypes = [_i64, _i64, _i64]
    L.mx_moe_dispatch.restype = ctypes.c_int
    L.mx_moe_dispatch_dual_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64,
                                               _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp]
    L.mx_moe_dispatch_dual_grouped.restype = ctypes.c_int
    L.mx_moe_combine.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp]
    L.mx_moe_combine.restype = ctypes.c_int
    L.mx_gemm.restype = ctypes.c_int
    L.mx_gemm.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                          ctypes.c_int, _vp, _i64, _vp]
    L.mx_gemm_workspace_bytes.restype = _i64
    L.mx_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int]
    L.mx_grouped_gemm.restype = ctypes.c_int
    L.mx_grouped_gemm.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                  _i64, ctypes.c_int, _vp]
    L.mx_quantize_dual_grouped.restype = ctypes.c_int
    L.mx_quantize_dual_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                                           _i64, _vp, _vp]
    L.mx_swiglu_quantize_dual_grouped.restype = ctypes.c_int
    L.mx_swiglu_quantize_dual_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp,
                                                  _i64, _i64, _vp, _vp]
    L.mx_quantize_rowwise_swz.restype = ctypes.c_int
    L.mx_quantize_rowwise_swz.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
    L.mx_quantize_colwise_swz.restype = ctypes.c_int
    L.mx_quantize_colwise_swz.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
    L.mx_quantize_rowwise_swz_batch.restype = ctypes.c_int
    L.mx_quantize_rowwise_swz_batch.argtypes = [ctypes.c_void_p, ctypes.c_int, _vp]
    L.mx_swiglu_quantize.restype = ctypes.c_int
    L.mx_swiglu_quantize.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]
    L.mx_quantize_dual_experts.restype = ctypes.c_int
    L.mx_quantize_dual_experts.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
    L.mx_grouped_k_capacity.restype = _i64
    L.mx_grouped_k_capacity.argtypes = [_i64, _i64]
    L.mx_quantize_colwise_grouped.restype = ctypes.c_int
    L.mx_quantize_colwise_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64,
                                              _i64, _vp, _vp]
    L.mx_grouped_gemm_wgrad.restype = ctypes.c_int
    L.mx_grouped_gemm_wgrad.argtypes = [_i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                                        _vp, _vp, _i64, ctypes.c_int, _vp, _i64, _vp]
    L.mx_grouped_gemm_wgrad_workspace_bytes.restype = _i64
    L.mx_grouped_gemm_wgrad_workspace_bytes.argtypes = []
    _lib = L
    return L


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> Tuple[int, int]:
    """(pointer, bytes) of the caller's workspace, or of a new uint8 tensor of
    the size the library asked for (the caller keeps ownership: the tensor is
    held by torch's allocator for the stream until the call's work is done)."""
    if need <= 0 and ws is None:
        return 0, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if not ws.is_cuda:
        raise ValueError("workspace must be a device tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _status_name(st: int) -> str:
    return load().mx_status_string(st).decode()


def _check(fn: str, st: int) -> None:
    if st != MX_OK:
        raise MxError(fn, st, load().mx_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _ld(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major view")
    return t.stride(0)


_BYTE_VIEWS = tuple(getattr(torch, n) for n in ("float8_e4m3fn", "float8_e8m0fnu")
                    if hasattr(torch, n))


def _u8(t: torch.Tensor) -> torch.Tensor:
    # E4M3 and E8M0 buffers are bytes at the ABI; accept float8 views too
    if t.dtype in _BYTE_VIEWS:
        return t.view(torch.uint8)
    return t


# ---------------------------------------------------------------------------


def mx_abi_version() -> int:
    return load().mx_abi_version()


def mx_status_string(status: int) -> str:
    return load().mx_status_string(status).decode()


def mx_last_error() -> str:
    """Message of the last non-MX_OK status returned on this thread."""
    return load().mx_last_error().decode()


def mx_scale_swizzled_bytes(rows: int, kblocks: int) -> int:
    return load().mx_scale_swizzled_bytes(rows, kblocks)


def mx_quantize_rowwise(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                        s: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """BF16 x[rows][cols] -> (q uint8 [rows][cols] E4M3, s uint8 [rows][cols/32] E8M0)."""
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    q, s = _u8(q), _u8(s)
    st = load().mx_quantize_rowwise(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                    _dev(q, "q", torch.uint8), _ld(q, "q"),
                                    _dev(s, "s", torch.uint8), _ld(s, "s"), _stream(stream))
    _check("mx_quantize_rowwise", st)
    return q, s


def mx_quantize_colwise(x: torch.Tensor, qt: Optional[torch.Tensor] = None,
                        st_: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """BF16 x[rows][cols] -> (qt uint8 [cols][rows], st uint8 [cols][rows/32]), transposed."""
    rows, cols = x.shape
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if st_ is None:
        st_ = torch.empty((cols, rows // 32), dtype=torch.uint8, device=x.device)
    qt, st_ = _u8(qt), _u8(st_)
    st = load().mx_quantize_colwise(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                    _dev(qt, "qt", torch.uint8), _ld(qt, "qt"),
                                    _dev(st_, "st", torch.uint8), _ld(st_, "st"),
                                    _stream(stream))
    _check("mx_quantize_colwise", st)
    return qt, st_


def mx_scale_swizzle(s: torch.Tensor, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """E8M0 s[rows][kblocks] -> the GEMM's rearranged scale buffer (uint8, 1-D)."""
    s = _u8(s)
    rows, kb = s.shape
    n = mx_scale_swizzled_bytes(rows, kb)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=s.device)
    if out.numel() < n:
        raise ValueError(f"out holds {out.numel()} bytes, needs {n}")
    st = load().mx_scale_swizzle(_dev(s, "s", torch.uint8), rows, kb, _ld(s, "s"),
                                 _dev(out, "out", torch.uint8), _stream(stream))
    _check("mx_scale_swizzle", st)
    return out


def mx_quantize_dual(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                     s_swz: Optional[torch.Tensor] = None, qt: Optional[torch.Tensor] = None,
                     st_swz: Optional[torch.Tensor] = None, s_tiles: Optional[int] = None,
                     st_tiles: Optional[int] = None, stream=None):
    """BF16 x[rows][cols] -> (q [rows][cols], s_swz, qt [cols][rows], st_swz): both
    orientations, scales in the GEMM's rearranged layout (see mx_quantize_dual in
    the header for s_tiles / st_tiles and writing into a larger buffer)."""
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if s_tiles is None:
        s_tiles = (cols // 32 + 7) // 8
    if st_tiles is None:
        st_tiles = (rows // 32 + 7) // 8
    if s_swz is None:
        s_swz = torch.empty(mx_scale_swizzled_bytes(rows, cols // 32), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(cols, rows // 32), dtype=torch.uint8, device=dev)
    q, qt, s_swz, st_swz = _u8(q), _u8(qt), _u8(s_swz), _u8(st_swz)
    st = load().mx_quantize_dual(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                 _dev(q, "q", torch.uint8), _ld(q, "q"),
                                 _dev(s_swz, "s_swz", torch.uint8), s_tiles,
                                 _dev(qt, "qt", torch.uint8), _ld(qt, "qt"),
                                 _dev(st_swz, "st_swz", torch.uint8), st_tiles, _stream(stream))
    _check("mx_quantize_dual", st)
    return q, s_swz, qt, st_swz


class _DualJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_x", ctypes.c_int64), ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64),
                ("s_swz", ctypes.c_void_p), ("s_tiles", ctypes.c_int64),
                ("qt", ctypes.c_void_p), ("ld_qt", ctypes.c_int64),
                ("st_swz", ctypes.c_void_p), ("st_tiles", ctypes.c_int64)]


def mx_quantize_dual_batch(jobs, stream=None) -> None:
    """Several dual quantizations in one launch.  jobs: a sequence of dicts with
    the device tensors x, q, s_swz, qt, st_swz and optionally s_tiles / st_tiles
    (the meaning of mx_quantize_dual's arguments); outputs are written in place."""
    arr = (_DualJob * max(len(jobs), 1))()
    for i, j in enumerate(jobs):
        x = j["x"]
        rows, cols = x.shape
        q, s_swz, qt, st_swz = (_u8(j[k]) for k in ("q", "s_swz", "qt", "st_swz"))
        arr[i] = _DualJob(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                          _dev(q, "q", torch.uint8), _ld(q, "q"),
                          _dev(s_swz, "s_swz", torch.uint8),
                          j.get("s_tiles", (cols // 32 + 7) // 8),
                          _dev(qt, "qt", torch.uint8), _ld(qt, "qt"),
                          _dev(st_swz, "st_swz", torch.uint8),
                          j.get("st_tiles", (rows // 32 + 7) // 8))
    st = load().mx_quantize_dual_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream))
    _check("mx_quantize_dual_batch", st)


def mx_moe_dispatch(x: torch.Tensor, topk_ids: torch.Tensor, num_experts: int,
                    offsets: Optional[torch.Tensor] = None, src: Optional[torch.Tensor] = None,
                    slot: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                    s_swz: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """Sort the routed rows by expert, gather and quantize them row-wise.

    x BF16 [tokens][hidden], topk_ids int32 [tokens][topk] -> (offsets int64
    [num_experts+1], src_token int32 [tokens*topk], slot int32 [tokens*topk],
    q uint8 [tokens*topk][hidden], s_swz uint8: rearranged scales); outputs
    passed in are written in place.  workspace: device scratch of at least
    mx_moe_dispatch_workspace_bytes bytes (a new tensor if None)."""
    tokens, hidden = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != tokens or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [tokens][topk] tensor")
    topk = topk_ids.shape[1]
    n = tokens * topk
    dev = x.device
    if offsets is None:
        offsets = torch.empty(num_experts + 1, dtype=torch.int64, device=dev)
    if src is None:
        src = torch.empty(n, dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty(n, dtype=torch.int32, device=dev)
    if q is None:
        q = torch.empty((n, hidden), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(mx_scale_swizzled_bytes(n, hidden // 32), dtype=torch.uint8, device=dev)
    if offsets.numel() != num_experts + 1 or src.numel() != n or slot.numel() != n:
        raise ValueError("offsets, src and slot must have num_experts+1, n and n entries")
    wp, wb = _workspace(workspace, mx_moe_dispatch_workspace_bytes(tokens, topk, num_experts), dev)
    st = load().mx_moe_dispatch(_dev(x, "x", torch.bfloat16), tokens, hidden, _ld(x, "x"),
                                _dev(topk_ids, "topk_ids", torch.int32), topk, num_experts,
                                _dev(offsets, "offsets"), _dev(src, "src"), _dev(slot, "slot"),
                                _dev(q, "q"), _ld(q, "q"), _dev(s_swz, "s_swz"), wp, wb, _stream(stream))
    _check("mx_moe_dispatch", st)
    return offsets, src, slot, q, s_swz


def mx_moe_dispatch_dual_grouped(x: torch.Tensor, topk_ids: torch.Tensor, num_experts: int,
                                 k_cap: Optional[int] = None, offsets: Optional[torch.Tensor] = None,
                                 src: Optional[torch.Tensor] = None, slot: Optional[torch.Tensor] = None,
                                 q: Optional[torch.Tensor] = None, s_swz: Optional[torch.Tensor] = None,
                                 pad_offsets: Optional[torch.Tensor] = None, qt: Optional[torch.Tensor] = None,
                                 st_swz: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                 stream=None):
    """mx_moe_dispatch that also quantizes the dispatched rows per expert
    column-wise (the gate_up weight gradient's operand) from the same reads.
    Returns (offsets, src_token, slot, q, s_swz, pad_offsets, qt [hidden][k_cap],
    st_swz); outputs passed in are written in place."""
    tokens, hidden = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != tokens or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [tokens][topk] tensor")
    topk = topk_ids.shape[1]
    n = tokens * topk
    dev = x.device
    if k_cap is None:
        k_cap = mx_grouped_k_capacity(n, num_experts)
    if offsets is None:
        offsets = torch.empty(num_experts + 1, dtype=torch.int64, device=dev)
    if src is None:
        src = torch.empty(n, dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty(n, dtype=torch.int32, device=dev)
    if q is None:
        q = torch.empty((n, hidden), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(mx_scale_swizzled_bytes(n, hidden // 32), dtype=torch.uint8, device=dev)
    if pad_offsets is None:
        pad_offsets = torch.empty(num_experts + 1, dtype=torch.int64, device=dev)
    if qt is None:
        qt = torch.empty((hidden, k_cap), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(hidden, k_cap // 32), dtype=torch.uint8, device=dev)
    if offsets.numel() != num_experts + 1 or src.numel() != n or slot.numel() != n:
        raise ValueError("offsets, src and slot must have num_experts+1, n and n entries")
    q, s_swz, qt, st_swz = _u8(q), _u8(s_swz), _u8(qt), _u8(st_swz)
    wp, wb = _workspace(workspace, mx_moe_dispatch_workspace_bytes(tokens, topk, num_experts), dev)
    st = load().mx_moe_dispatch_dual_grouped(
        _dev(x, "x", torch.bfloat16), tokens, hidden, _ld(x, "x"), _dev(topk_ids, "topk_ids", torch.int32), topk,
        num_experts, _dev(offsets, "offsets"), _dev(src, "src"), _dev(slot, "slot"), _dev(q, "q"), _ld(q, "q"),
        _dev(s_swz, "s_swz"), _dev(pad_offsets, "pad_offsets", torch.int64), _dev(qt, "qt"), _ld(qt, "qt"), k_cap,
        _dev(st_swz, "st_swz"), wp, wb, _stream(stream))
    _check("mx_moe_dispatch_dual_grouped", st)
    return offsets, src, slot, q, s_swz, pad_offsets, qt, st_swz


def mx_moe_dispatch_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, num_experts: int,
                            offsets: torch.Tensor, src: torch.Tensor, slot: torch.Tensor,
                            q: torch.Tensor, s_swz: torch.Tensor, stream=None):
    """mx_moe_dispatch without a workspace (its chunk counts in the library's
    device array): every output is passed in, so the call allocates nothing."""
    tokens, hidden = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != tokens or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [tokens][topk] tensor")
    topk = topk_ids.shape[1]
    n = tokens * topk
    if offsets.numel() != num_experts + 1 or src.numel() != n or slot.numel() != n:
        raise ValueError("offsets, src and slot must have num_experts+1, n and n entries")
    st = load().mx_moe_dispatch_noalloc(_dev(x, "x", torch.bfloat16), tokens, hidden, _ld(x, "x"),
                                        _dev(topk_ids, "topk_ids", torch.int32), topk, num_experts,
                                        _dev(offsets, "offsets", torch.int64), _dev(src, "src", torch.int32),
                                        _dev(slot, "slot", torch.int32), _dev(_u8(q), "q", torch.uint8),
                                        _ld(q, "q"), _dev(_u8(s_swz), "s_swz", torch.uint8), _stream(stream))
    _check("mx_moe_dispatch_noalloc", st)
    return offsets, src, slot, q, s_swz


def mx_moe_combine(y: torch.Tensor, slot: torch.Tensor, weights: torch.Tensor,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[t] = sum_j weights[t][j] * y[slot[t*topk + j]] (BF16 [tokens][hidden])."""
    tokens, topk = weights.shape
    hidden = y.shape[1]
    if out is None:
        out = torch.empty((tokens, hidden), dtype=torch.bfloat16, device=y.device)
    if not (slot.is_contiguous() and weights.is_contiguous()):
        raise ValueError("slot and weights must be contiguous")
    st = load().mx_moe_combine(_dev(y, "y", torch.bfloat16), tokens, hidden, _ld(y, "y"),
                               _dev(slot, "slot", torch.int32), _dev(weights, "weights", torch.float32),
                               topk, _dev(out, "out", torch.bfloat16), _ld(out, "out"), _stream(stream))
    _check("mx_moe_combine", st)
    return out


_OUT = {torch.bfloat16: MX_BF16, torch.float32: MX_F32}


def mx_gemm_workspace_bytes(M: int, N: int, K: int, out_dtype: torch.dtype = torch.bfloat16) -> int:
    """Device scratch mx_gemm needs for this shape (0: none), host-only."""
    return load().mx_gemm_workspace_bytes(M, N, K, _OUT[out_dtype])


def mx_moe_dispatch_workspace_bytes(tokens: int, topk: int, num_experts: int) -> int:
    return load().mx_moe_dispatch_workspace_bytes(tokens, topk, num_experts)


def mx_grouped_gemm_wgrad_workspace_bytes() -> int:
    return load().mx_grouped_gemm_wgrad_workspace_bytes()


def mx_gemm(a_q: torch.Tensor, a_s_swz: torch.Tensor, b_q: torch.Tensor,
            b_s_swz: torch.Tensor, c: Optional[torch.Tensor] = None,
            out_dtype: torch.dtype = torch.bfloat16, workspace: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """C[M][N] = deq(A)[M][K] . deq(B)[N][K]^T (both operands K-contiguous).
    workspace: device scratch of at least mx_gemm_workspace_bytes bytes when
    that is nonzero (a new tensor if None)."""
    a_q, b_q = _u8(a_q), _u8(b_q)
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError(f"K mismatch: A {tuple(a_q.shape)} B {tuple(b_q.shape)}")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    if c.dtype not in _OUT:
        raise ValueError("c must be bfloat16 or float32")
    wp, wb = _workspace(workspace, mx_gemm_workspace_bytes(M, N, K, c.dtype), a_q.device)
    st = load().mx_gemm(M, N, K, _dev(a_q, "a_q", torch.uint8), _ld(a_q, "a_q"),
                        _dev(a_s_swz, "a_s_swz", torch.uint8), _dev(b_q, "b_q", torch.uint8),
                        _ld(b_q, "b_q"), _dev(b_s_swz, "b_s_swz", torch.uint8),
                        _dev(c, "c"), _ld(c, "c"), _OUT[c.dtype], wp, wb, _stream(stream))
    _check("mx_gemm", st)
    return c


def mx_grouped_gemm(group_offsets: torch.Tensor, a_q: torch.Tensor, a_s_swz: torch.Tensor,
                    b_q: torch.Tensor, b_s_swz: torch.Tensor, c: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Per-expert C: rows [off[g], off[g+1]) of A times B_g^T, B as [G][N][K]."""
    a_q, b_q = _u8(a_q), _u8(b_q)
    M, K = a_q.shape
    G, N, Kb = b_q.shape
    if Kb != K:
        raise ValueError(f"K mismatch: A {tuple(a_q.shape)} B {tuple(b_q.shape)}")
    if not b_q.is_contiguous():
        raise ValueError("b_q must be contiguous [G][N][K]")
    if group_offsets.dtype != torch.int64 or group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must be int64 with G+1 entries")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    if c.dtype not in _OUT:
        raise ValueError("c must be bfloat16 or float32")
    st = load().mx_grouped_gemm(G, M, N, K, _dev(group_offsets, "group_offsets"),
                                _dev(a_q, "a_q", torch.uint8), _ld(a_q, "a_q"),
                                _dev(a_s_swz, "a_s_swz", torch.uint8),
                                _dev(b_q, "b_q", torch.uint8),
                                _dev(b_s_swz, "b_s_swz", torch.uint8), _dev(c, "c"),
                                _ld(c, "c"), _OUT[c.dtype], _stream(stream))
    _check("mx_grouped_gemm", st)
    return c


def mx_quantize_dual_experts(w: torch.Tensor, q: Optional[torch.Tensor] = None,
                             s_swz: Optional[torch.Tensor] = None, qt: Optional[torch.Tensor] = None,
                             st_swz: Optional[torch.Tensor] = None, stream=None):
    """Stacked expert weights w [G][N][K] (BF16) -> (q [G][N][K], s_swz, qt [G][K][N],
    st_swz): each expert quantized row-wise and column-wise in one launch, its
    rearranged scales back to back (expert g at g * mx_scale_swizzled_bytes of
    one expert), the layouts mx_grouped_gemm takes for B."""
    G, N, K = w.shape
    dev = w.device
    if not w.is_contiguous():
        raise ValueError("w must be a contiguous [G][N][K] stack")
    if q is None:
        q = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    if qt is None:
        qt = torch.empty((G, K, N), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(G * mx_scale_swizzled_bytes(N, K // 32), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(G * mx_scale_swizzled_bytes(K, N // 32), dtype=torch.uint8, device=dev)
    q, qt, s_swz, st_swz = _u8(q), _u8(qt), _u8(s_swz), _u8(st_swz)
    for t, name in ((q, "q"), (qt, "qt")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    st = load().mx_quantize_dual_experts(_dev(w, "w", torch.bfloat16), G, N, K,
                                         _dev(q, "q", torch.uint8), _dev(s_swz, "s_swz", torch.uint8),
                                         _dev(qt, "qt", torch.uint8),
                                         _dev(st_swz, "st_swz", torch.uint8), _stream(stream))
    _check("mx_quantize_dual_experts", st)
    return q, s_swz, qt, st_swz


def mx_grouped_k_capacity(rows_total: int, num_groups: int) -> int:
    """Columns that hold every expert's 256-aligned range for any split of the rows."""
    return load().mx_grouped_k_capacity(rows_total, num_groups)


def mx_quantize_colwise_grouped(x: torch.Tensor, group_offsets: torch.Tensor,
                                k_cap: Optional[int] = None, qt: Optional[torch.Tensor] = None,
                                st_swz: Optional[torch.Tensor] = None,
                                pad_offsets: Optional[torch.Tensor] = None, stream=None):
    """x [rows][cols] BF16, rows sorted by expert -> (qt [cols][k_cap], st_swz,
    pad_offsets int64 [G+1]): per-expert column-wise quantization into 256-aligned
    column ranges (see mx_quantize_colwise_grouped in the header)."""
    rows, cols = x.shape
    G = group_offsets.numel() - 1
    if group_offsets.dtype != torch.int64 or G < 1:
        raise ValueError("group_offsets must be int64 with G+1 entries, G >= 1")
    if k_cap is None:
        k_cap = mx_grouped_k_capacity(rows, G)
    dev = x.device
    if qt is None:
        qt = torch.empty((cols, k_cap), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(cols, k_cap // 32), dtype=torch.uint8,
                             device=dev)
    if pad_offsets is None:
        pad_offsets = torch.empty(G + 1, dtype=torch.int64, device=dev)
    qt, st_swz = _u8(qt), _u8(st_swz)
    st = load().mx_quantize_colwise_grouped(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                            _dev(group_offsets, "group_offsets", torch.int64), G,
                                            _dev(pad_offsets, "pad_offsets", torch.int64),
                                            _dev(qt, "qt", torch.uint8), _ld(qt, "qt"), k_cap,
                                            _dev(st_swz, "st_swz", torch.uint8), _stream(stream))
    _check("mx_quantize_colwise_grouped", st)
    return qt, st_swz, pad_offsets


def mx_grouped_gemm_wgrad(k_offsets: torch.Tensor, a_q: torch.Tensor, a_s_swz: torch.Tensor,
                          b_q: torch.Tensor, b_s_swz: torch.Tensor, c: Optional[torch.Tensor] = None,
                          out_dtype: torch.dtype = torch.bfloat16, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """C [G][M][N]: C_g = A[:, r_g] B[:, r_g]^T over the column ranges
    r_g = [k_offsets[g], k_offsets[g+1]) (the per-expert weight gradient).
    workspace: mx_grouped_gemm_wgrad_workspace_bytes() bytes of device scratch
    (a new tensor if None)."""
    a_q, b_q = _u8(a_q), _u8(b_q)
    M, K = a_q.shape
    N, Kb = b_q.shape
    if Kb != K:
        raise ValueError(f"K mismatch: A {tuple(a_q.shape)} B {tuple(b_q.shape)}")
    G = k_offsets.numel() - 1
    if k_offsets.dtype != torch.int64 or G < 1:
        raise ValueError("k_offsets must be int64 with G+1 entries, G >= 1")
    if c is None:
        c = torch.empty((G, M, N), dtype=out_dtype, device=a_q.device)
    if c.dtype not in _OUT:
        raise ValueError("c must be bfloat16 or float32")
    if c.dim() != 3 or c.shape[0] != G or c.shape[1] != M or c.stride(2) != 1 or \
            c.stride(0) != M * c.stride(1):
        raise ValueError("c must be [G][M][ld_c] with row-major experts back to back")
    st = load().mx_grouped_gemm_wgrad(G, M, N, K, _dev(k_offsets, "k_offsets", torch.int64),
                                      _dev(a_q, "a_q", torch.uint8), _ld(a_q, "a_q"),
                                      _dev(a_s_swz, "a_s_swz", torch.uint8),
                                      _dev(b_q, "b_q", torch.uint8), _ld(b_q, "b_q"),
                                      _dev(b_s_swz, "b_s_swz", torch.uint8), _dev(c, "c"),
                                      c.stride(1), _OUT[c.dtype],
                                      *_workspace(workspace, mx_grouped_gemm_wgrad_workspace_bytes(), a_q.device),
                                      _stream(stream))
    _check("mx_grouped_gemm_wgrad", st)
    return c


def mx_swiglu_quantize(gu: torch.Tensor, q: Optional[torch.Tensor] = None,
                       s_swz: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None,
                       want_h: bool = False, stream=None):
    """gu [rows][2F] BF16 (gate | up) -> (q [rows][F], s_swz, h or None): SwiGLU,
    rounded to BF16, quantized row-wise with scales in the GEMM layout."""
    rows, F2 = gu.shape
    F = F2 // 2
    dev = gu.device
    if q is None:
        q = torch.empty((rows, F), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(mx_scale_swizzled_bytes(rows, F // 32), dtype=torch.uint8, device=dev)
    if h is None and want_h:
        h = torch.empty((rows, F), dtype=torch.bfloat16, device=dev)
    q, s_swz = _u8(q), _u8(s_swz)
    st = load().mx_swiglu_quantize(_dev(gu, "gu", torch.bfloat16), rows, F, _ld(gu, "gu"),
                                   _dev(h, "h", torch.bfloat16) if h is not None else None,
                                   _ld(h, "h") if h is not None else 0,
                                   _dev(q, "q", torch.uint8), _ld(q, "q"),
                                   _dev(s_swz, "s_swz", torch.uint8), _stream(stream))
    _check("mx_swiglu_quantize", st)
    return q, s_swz, h


def mx_quantize_rowwise_swz(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                            s_swz: Optional[torch.Tensor] = None, s_tiles: Optional[int] = None,
                            stream=None):
    """BF16 x[rows][cols] -> (q [rows][cols], s_swz): row-wise MXFP8 with the scales
    stored in the GEMM's rearranged layout in the same pass."""
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if s_tiles is None:
        s_tiles = cols // 256
    if s_swz is None:
        s_swz = torch.empty(mx_scale_swizzled_bytes(rows, cols // 32), dtype=torch.uint8, device=dev)
    q, s_swz = _u8(q), _u8(s_swz)
    st = load().mx_quantize_rowwise_swz(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                        _dev(q, "q", torch.uint8), _ld(q, "q"),
                                        _dev(s_swz, "s_swz", torch.uint8), s_tiles, _stream(stream))
    _check("mx_quantize_rowwise_swz", st)
    return q, s_swz


class _RowJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_x", ctypes.c_int64), ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64),
                ("s_swz", ctypes.c_void_p), ("s_tiles", ctypes.c_int64)]


def mx_quantize_rowwise_swz_batch(jobs, stream=None) -> None:
    """Several mx_quantize_rowwise_swz in one launch.  jobs: a sequence of dicts
    with the device tensors x, q, s_swz and optionally s_tiles (the meaning of
    mx_quantize_rowwise_swz's arguments); outputs are written in place."""
    arr = (_RowJob * max(len(jobs), 1))()
    for i, j in enumerate(jobs):
        x = j["x"]
        rows, cols = x.shape
        q, s_swz = _u8(j["q"]), _u8(j["s_swz"])
        arr[i] = _RowJob(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                         _dev(q, "q", torch.uint8), _ld(q, "q"),
                         _dev(s_swz, "s_swz", torch.uint8), j.get("s_tiles", cols // 256))
    st = load().mx_quantize_rowwise_swz_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream))
    _check("mx_quantize_rowwise_swz_batch", st)


def mx_quantize_colwise_swz(x: torch.Tensor, qt: Optional[torch.Tensor] = None,
                            st_swz: Optional[torch.Tensor] = None, st_tiles: Optional[int] = None,
                            stream=None):
    """BF16 x[rows][cols] -> (qt [cols][rows], st_swz): column-wise MXFP8,
    transposed, with the scales stored in the GEMM's rearranged layout."""
    rows, cols = x.shape
    dev = x.device
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if st_tiles is None:
        st_tiles = rows // 256
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(cols, rows // 32), dtype=torch.uint8, device=dev)
    qt, st_swz = _u8(qt), _u8(st_swz)
    st = load().mx_quantize_colwise_swz(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                        _dev(qt, "qt", torch.uint8), _ld(qt, "qt"),
                                        _dev(st_swz, "st_swz", torch.uint8), st_tiles, _stream(stream))
    _check("mx_quantize_colwise_swz", st)
    return qt, st_swz


def mx_quantize_dual_grouped(x: torch.Tensor, group_offsets: torch.Tensor, k_cap: Optional[int] = None,
                             q: Optional[torch.Tensor] = None, s_swz: Optional[torch.Tensor] = None,
                             qt: Optional[torch.Tensor] = None, st_swz: Optional[torch.Tensor] = None,
                             pad_offsets: Optional[torch.Tensor] = None, stream=None):
    """x [rows][cols] BF16, rows sorted by expert -> (q [rows][cols], s_swz, qt
    [cols][k_cap], st_swz, pad_offsets): row-wise and per-expert column-wise
    quantization from one read (see mx_quantize_dual_grouped in the header)."""
    rows, cols = x.shape
    G = group_offsets.numel() - 1
    if group_offsets.dtype != torch.int64 or G < 1:
        raise ValueError("group_offsets must be int64 with G+1 entries, G >= 1")
    if k_cap is None:
        k_cap = mx_grouped_k_capacity(rows, G)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(max(mx_scale_swizzled_bytes(rows, cols // 32), 1), dtype=torch.uint8, device=dev)
    if qt is None:
        qt = torch.empty((cols, k_cap), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(cols, k_cap // 32), dtype=torch.uint8, device=dev)
    if pad_offsets is None:
        pad_offsets = torch.empty(G + 1, dtype=torch.int64, device=dev)
    q, s_swz, qt, st_swz = _u8(q), _u8(s_swz), _u8(qt), _u8(st_swz)
    st = load().mx_quantize_dual_grouped(_dev(x, "x", torch.bfloat16), rows, cols, _ld(x, "x"),
                                         _dev(group_offsets, "group_offsets", torch.int64), G,
                                         _dev(pad_offsets, "pad_offsets", torch.int64),
                                         _dev(q, "q", torch.uint8), _ld(q, "q"),
                                         _dev(s_swz, "s_swz", torch.uint8),
                                         _dev(qt, "qt", torch.uint8), _ld(qt, "qt"), k_cap,
                                         _dev(st_swz, "st_swz", torch.uint8), _stream(stream))
    _check("mx_quantize_dual_grouped", st)
    return q, s_swz, qt, st_swz, pad_offsets


def mx_swiglu_quantize_dual_grouped(gu: torch.Tensor, group_offsets: torch.Tensor, k_cap: Optional[int] = None,
                                    q: Optional[torch.Tensor] = None, s_swz: Optional[torch.Tensor] = None,
                                    qt: Optional[torch.Tensor] = None, st_swz: Optional[torch.Tensor] = None,
                                    pad_offsets: Optional[torch.Tensor] = None, stream=None):
    """gu [rows][2F] BF16 (gate, then up), rows sorted by expert -> (q [rows][F],
    s_swz, qt [F][k_cap], st_swz, pad_offsets): h = SwiGLU(gate, up) quantized
    row-wise and per expert column-wise from one read, h never written (see
    mx_swiglu_quantize_dual_grouped in the header)."""
    rows, two_f = gu.shape
    F = two_f // 2
    G = group_offsets.numel() - 1
    if group_offsets.dtype != torch.int64 or G < 1:
        raise ValueError("group_offsets must be int64 with G+1 entries, G >= 1")
    if k_cap is None:
        k_cap = mx_grouped_k_capacity(rows, G)
    dev = gu.device
    if q is None:
        q = torch.empty((rows, F), dtype=torch.uint8, device=dev)
    if s_swz is None:
        s_swz = torch.empty(max(mx_scale_swizzled_bytes(rows, F // 32), 1), dtype=torch.uint8, device=dev)
    if qt is None:
        qt = torch.empty((F, k_cap), dtype=torch.uint8, device=dev)
    if st_swz is None:
        st_swz = torch.empty(mx_scale_swizzled_bytes(F, k_cap // 32), dtype=torch.uint8, device=dev)
    if pad_offsets is None:
        pad_offsets = torch.empty(G + 1, dtype=torch.int64, device=dev)
    q, s_swz, qt, st_swz = _u8(q), _u8(s_swz), _u8(qt), _u8(st_swz)
    st = load().mx_swiglu_quantize_dual_grouped(_dev(gu, "gu", torch.bfloat16), rows, F, _ld(gu, "gu"),
                                                _dev(group_offsets, "group_offsets", torch.int64), G,
                                                _dev(pad_offsets, "pad_offsets", torch.int64),
                                                _dev(q, "q", torch.uint8), _ld(q, "q"),
                                                _dev(s_swz, "s_swz", torch.uint8),
                                                _dev(qt, "qt", torch.uint8), _ld(qt, "qt"), k_cap,
                                                _dev(st_swz, "st_swz", torch.uint8), _stream(stream))
    _check("mx_swiglu_quantize_dual_grouped", st)
    return q, s_swz, qt, st_swz, pad_offsets
