"""Run inside a process that preloads the AddressSanitizer runtime (see
tests/test_sanitize_cpu.py): the oracle's pin tests against the sanitized
oracle build, the C-ABI tests against the sanitized validation layer, then
every entry point called with VALID arguments (fake device addresses that
the stub launchers never touch), at small and at near-limit sizes, so the
validation arithmetic runs to the launch on each."""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))
sys.path.insert(0, HERE)

import build  # noqa: E402

ORACLE_LIB, API_LIB = build.ORACLE_LIB, build.API_LIB

import oracle  # noqa: E402
import mxfp8_block_scaled_08_amd as mx  # noqa: E402

oracle.LIB = ORACLE_LIB
mx._LIB_PATH = API_LIB

import pytest  # noqa: E402

rc = pytest.main(["-q", "-p", "no:cacheprovider", "-x", "-m", "not gpu",
                  os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                  os.path.join(ROOT, "tests", "test_oracle_moe_pins.py"),
                  os.path.join(ROOT, "tests", "test_oracle_moe_bwd_pins.py"),
                  os.path.join(ROOT, "tests", "test_oracle_swiglu_pins.py"),
                  os.path.join(ROOT, "tests", "test_oracle_agreement.py"),
                  os.path.join(ROOT, "tests", "test_mfma_model_cpu.py"),
                  os.path.join(ROOT, "tests", "test_abi_cpu.py")])
if rc != 0:
    sys.exit(int(rc))
assert oracle.lib()._name == ORACLE_LIB and mx.load()._name == API_LIB

L = ctypes.CDLL(API_LIB)
launches = ctypes.c_int64.in_dll(L, "stub_launches")
last_ws = ctypes.c_int64.in_dll(L, "stub_last_ws")
I, V = ctypes.c_int64, ctypes.c_void_p
A0, A1, A2, A3, A4, A5, WS = (1 << 40), (2 << 40), (3 << 40), (4 << 40), (5 << 40), (6 << 40), (7 << 40)


def ok(fn, *args):
    before = launches.value
    st = getattr(L, fn)(*args)
    msg = ctypes.c_char_p(L.mx_last_error()).value
    assert st == 0, (fn, st, msg)
    assert launches.value == before + 1, fn


for name in ("mx_quantize_rowwise", "mx_quantize_colwise"):
    f = getattr(L, name)
    f.argtypes = [V, I, I, I, V, I, V, I, V]
L.mx_last_error.restype = ctypes.c_void_p
for rows, cols in ((1, 32), (4096, 4096), (1 << 20, 1 << 14)):
    ok("mx_quantize_rowwise", A0, rows, cols, cols, A1, cols, A2, cols // 32, None)
    ok("mx_quantize_colwise", A0, rows * 32, cols, cols, A1, rows * 32, A2, rows, None)
L.mx_quantize_rowwise_swz.argtypes = [V, I, I, I, V, I, V, I, V]
ok("mx_quantize_rowwise_swz", A0, 163840, 2048, 2048, A1, 2048, A2, 8, None)
L.mx_scale_swizzle.argtypes = [V, I, I, I, V, V]
ok("mx_scale_swizzle", A0, 12288, 384, 384, A1, None)
L.mx_quantize_dual.argtypes = [V, I, I, I, V, I, V, I, V, I, V, I, V]
ok("mx_quantize_dual", A0, 12288, 24576, 24576, A1, 24576, A2, 96, A3, 12288, A4, 48, None)
L.mx_quantize_dual_experts.argtypes = [V, I, I, I, V, V, V, V, V]
ok("mx_quantize_dual_experts", A0, 128, 1536, 2048, A1, A2, A3, A4, None)
L.mx_gemm.argtypes = [I, I, I, V, I, V, V, I, V, V, I, ctypes.c_int, V, I, V]
L.mx_gemm_workspace_bytes.restype = I
L.mx_gemm_workspace_bytes.argtypes = [I, I, I, ctypes.c_int]
for M, N, K in ((128, 256, 256), (4608, 4096, 4096), (4608, 6144, 4096), (12288, 4096, 24576),
                (1 << 20, 1 << 16, 1 << 12), (4608, 4096, 12288)):
    need = L.mx_gemm_workspace_bytes(M, N, K, 0)
    ok("mx_gemm", M, N, K, A0, K, A1, A2, K, A3, A4, N, 0, WS, need, None)
    assert last_ws.value == WS
L.mx_grouped_gemm.argtypes = [I, I, I, I, V, V, I, V, V, V, V, I, ctypes.c_int, V]
ok("mx_grouped_gemm", 128, 163840, 1536, 2048, A0, A1, 2048, A2, A3, A4, A5, 1536, 0, None)
L.mx_moe_dispatch.argtypes = [V, I, I, I, V, I, I, V, V, V, V, I, V, V, I, V]
L.mx_moe_dispatch_workspace_bytes.restype = I
L.mx_moe_dispatch_workspace_bytes.argtypes = [I, I, I]
need = L.mx_moe_dispatch_workspace_bytes(20480, 8, 128)
ok("mx_moe_dispatch", A0, 20480, 2048, 2048, A1, 8, 128, A2, A2 + (1 << 20), A2 + (2 << 20), A3, 2048, A4,
   WS, need, None)
L.mx_moe_dispatch_noalloc.argtypes = [V, I, I, I, V, I, I, V, V, V, V, I, V, V]
ok("mx_moe_dispatch_noalloc", A0, 20480, 2048, 2048, A1, 8, 128, A2, A2 + (1 << 20), A2 + (2 << 20), A3, 2048,
   A4, None)
L.mx_moe_combine.argtypes = [V, I, I, I, V, V, I, V, I, V]
ok("mx_moe_combine", A0, 20480, 2048, 2048, A1, A2, 8, A3, 2048, None)
L.mx_swiglu_quantize.argtypes = [V, I, I, I, V, I, V, I, V, V]
ok("mx_swiglu_quantize", A0, 163840, 768, 1536, A1, 768, A2, 768, A3, None)
L.mx_grouped_k_capacity.restype = I
L.mx_grouped_k_capacity.argtypes = [I, I]
kc = L.mx_grouped_k_capacity(163840, 128)
L.mx_quantize_colwise_grouped.argtypes = [V, I, I, I, V, I, V, V, I, I, V, V]
ok("mx_quantize_colwise_grouped", A0, 163840, 2048, 2048, A1, 128, A1 + 4096, A2, kc, kc, A3, None)
L.mx_quantize_dual_grouped.argtypes = [V, I, I, I, V, I, V, V, I, V, V, I, I, V, V]
ok("mx_quantize_dual_grouped", A0, 163840, 2048, 2048, A1, 128, A1 + 4096, A2, 2048, A3, A4, kc, kc, A5, None)
L.mx_grouped_gemm_wgrad.argtypes = [I, I, I, I, V, V, I, V, V, I, V, V, I, ctypes.c_int, V, I, V]
ok("mx_grouped_gemm_wgrad", 128, 1536, 2048, kc, A0, A1, kc, A2, A3, kc, A4, A5, 2048, 0, WS, 256, None)
assert last_ws.value == WS
print("sanitized valid calls:", launches.value, "launches reached")
