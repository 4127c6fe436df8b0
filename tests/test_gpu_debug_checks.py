"""The MX_DEBUG checks of device-resident offsets.

Normally the grouped entry points never read their offsets on the host: the
kernels clamp them, so offsets that break their stated properties give
unspecified but in-bounds results (tests/test_gpu_moe_bwd.py covers that).
With MX_DEBUG set, each of them first checks the offsets on the device,
waits for the check and returns MX_ERR_INVALID_ARG naming the first bad
entry, launching nothing, so the outputs keep their bytes.  Valid offsets
give the same bytes with and without the check."""
import numpy as np
import pytest
import torch

import mxsynth

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env(monkeypatch):
    monkeypatch.setenv("MX_DEBUG", "1")


def test_grouped_gemm_offsets_checked(gpu_lib, monkeypatch):
    mx = gpu_lib
    G, M, N, K = 3, 600, 256, 256
    x = mxsynth.normal_bf16((M, K), 1.0, seed=31).cuda()
    w = mxsynth.normal_bf16((G, N, K), 0.05, seed=32).cuda()
    aq, as_ = mx.mx_quantize_rowwise_swz(x)
    wq, ws, _, _ = mx.mx_quantize_dual_experts(w)
    good = torch.tensor([0, 100, 350, M], dtype=torch.int64, device="cuda")
    ref = mx.mx_grouped_gemm(good, aq, as_, wq, ws)
    monkeypatch.setenv("MX_DEBUG", "1")
    again = mx.mx_grouped_gemm(good, aq, as_, wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), again.view(torch.int16))
    for bad, idx in (([0, 350, 100, M], 1),      # decreasing
                     ([5, 100, 350, M], 0),      # not starting at 0
                     ([0, 100, 350, M - 1], 3),  # not ending at M
                     ([0, 100, 700, M], 2)):     # outside [0, M]
        c = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(mx.MxError) as e:
            mx.mx_grouped_gemm(torch.tensor(bad, dtype=torch.int64, device="cuda"), aq, as_, wq, ws, c=c)
        msg = str(e.value)
        assert "MX_DEBUG" in msg and f"group_offsets[{idx}]" in msg, msg
        torch.cuda.synchronize()
        assert (c == 3.0).all(), "an output was written after a failed check"
    monkeypatch.delenv("MX_DEBUG")
    # without the check the same offsets run (clamped, unspecified results)
    mx.mx_grouped_gemm(torch.tensor([0, 350, 100, M], dtype=torch.int64, device="cuda"), aq, as_, wq, ws)
    torch.cuda.synchronize()


def test_grouped_quantizer_and_wgrad_offsets_checked(gpu_lib, debug_env):
    mx = gpu_lib
    rows, cols, G = 700, 64, 3
    x = mxsynth.normal_bf16((rows, cols), 1.0, seed=41).cuda()
    k_cap = mx.mx_grouped_k_capacity(rows, G)
    good = torch.tensor([0, 200, 200, rows], dtype=torch.int64, device="cuda")
    qt, st, pad = mx.mx_quantize_colwise_grouped(x, good, k_cap=k_cap)
    c = mx.mx_grouped_gemm_wgrad(pad, qt, st, qt, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    # rows outside [0, rows], and a decreasing pair
    for bad, idx in (([0, 200, 100, rows], 1), ([0, 200, 300, rows + 1], 3)):
        qt2 = torch.full_like(qt, 0x33)
        with pytest.raises(mx.MxError) as e:
            mx.mx_quantize_colwise_grouped(x, torch.tensor(bad, dtype=torch.int64, device="cuda"), k_cap=k_cap,
                                           qt=qt2)
        assert f"group_offsets[{idx}]" in str(e.value), str(e.value)
        torch.cuda.synchronize()
        assert (qt2 == 0x33).all()
    # the one-read row-wise + per-expert column-wise form checks the same way
    x2 = mxsynth.normal_bf16((rows, 256), 1.0, seed=42).cuda()
    q2 = torch.full((rows, 256), 0x44, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError) as e:
        mx.mx_quantize_dual_grouped(x2, torch.tensor([0, 200, 100, rows], dtype=torch.int64, device="cuda"),
                                    k_cap=k_cap, q=q2)
    assert "mx_quantize_dual_grouped" in str(e.value) and "group_offsets[1]" in str(e.value), str(e.value)
    torch.cuda.synchronize()
    assert (q2 == 0x44).all()
    mx.mx_quantize_dual_grouped(x2, good, k_cap=k_cap, q=q2)
    torch.cuda.synchronize()
    # weight-gradient ranges: not 256-aligned, shorter than 256, past k_cap
    for bad, idx in (([0, 256, 600, 1024], 2), ([0, 256, 256, 768], 1), ([0, 256, 512, k_cap + 256], 3)):
        c2 = torch.full_like(c, 5.0)
        with pytest.raises(mx.MxError) as e:
            mx.mx_grouped_gemm_wgrad(torch.tensor(bad, dtype=torch.int64, device="cuda"), qt, st, qt, st, c=c2)
        assert f"k_offsets[{idx}]" in str(e.value), str(e.value)
        torch.cuda.synchronize()
        assert (c2 == 5.0).all()
