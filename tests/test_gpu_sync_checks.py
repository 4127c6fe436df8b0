"""Weight-synchronization checks as tests over the library.

The pages check each synchronization two ways ("End-to-End MXFP8
Reinforcement Learning on Blackwell", Table 11: a self-check through the
sampler's kernels and an offline byte comparison of the synchronized weights;
Table 13: a failure visible only in one expert or a late layer).  Here:
  - byte comparison: a layer synchronized the way bench.py does it (one
    batched dual-orientation pass) equals, byte for byte, a fresh
    re-quantization of the same weights by the separate quantizers and the
    rearrangement (values and scales); at a second synchronization a changed
    weight changes exactly the blocks that hold the change, and the copy
    taken at the first one no longer matches (a stale copy is visible);
  - probe GEMM on every expert: the MoE weights are quantized, their
    rearranged scales rebuilt per expert, and a grouped GEMM with one probe
    row per expert is checked against the oracle over all of every expert's
    output columns; a stale rearranged scale copy of a single expert shows up
    in that expert's row and nowhere else."""
import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import (assert_gemm_close, bf16_dev, grouped_ref, oracle_rowwise_par)

pytestmark = pytest.mark.gpu


def _sync(mx, W):
    """Both orientations of every weight, scales rearranged, one launch."""
    out, jobs = {}, []
    for n, w in W.items():
        r, c = w.shape
        o = dict(x=w, q=torch.empty((r, c), dtype=torch.uint8, device="cuda"),
                 s_swz=torch.empty((mx.mx_scale_swizzled_bytes(r, c // 32),), dtype=torch.uint8,
                                   device="cuda"),
                 qt=torch.empty((c, r), dtype=torch.uint8, device="cuda"),
                 st_swz=torch.empty((mx.mx_scale_swizzled_bytes(c, r // 32),), dtype=torch.uint8,
                                    device="cuda"))
        out[n] = o
        jobs.append(o)
    mx.mx_quantize_dual_batch(jobs)
    return {n: (o["q"], o["s_swz"], o["qt"], o["st_swz"]) for n, o in out.items()}


def _requantize(mx, w):
    q, s = mx.mx_quantize_rowwise(w)
    qt, st = mx.mx_quantize_colwise(w)
    return q, mx.mx_scale_swizzle(s), qt, mx.mx_scale_swizzle(st)


def test_sync_byte_comparison_two_synchronizations(gpu_lib):
    mx = gpu_lib
    W = {n: w.cuda() for n, w in mxsynth.weight_sync().items()}
    synced = _sync(mx, W)
    torch.cuda.synchronize()
    for n, w in W.items():
        for got, ref, what in zip(synced[n], _requantize(mx, w), ("q", "s_swz", "qt", "st_swz")):
            assert torch.equal(got, ref), f"sync 1: {n} {what} differs from a re-quantization"
    # the synchronized bytes of one weight against the oracle
    oq, os_ = oracle_rowwise_par(mxsynth.bits(W["k"].cpu()))
    assert np.array_equal(synced["k"][0].cpu().numpy(), oq)
    assert np.array_equal(synced["k"][1].cpu().numpy(), oracle.scale_swizzle(os_))

    # second synchronization: an update touching rows 100..131 of o, one element of down
    W2 = {n: w.clone() for n, w in W.items()}
    W2["o"][100:132] *= 3.0
    W2["down"][7, 4000] = 1.5
    synced2 = _sync(mx, W2)
    for n, w in W2.items():
        for got, ref, what in zip(synced2[n], _requantize(mx, w), ("q", "s_swz", "qt", "st_swz")):
            assert torch.equal(got, ref), f"sync 2: {n} {what} differs from a re-quantization"
    for n in W:
        same = all(torch.equal(a, b) for a, b in zip(synced[n], synced2[n]))
        assert same == (n not in ("o", "down")), f"{n}: bytes {'unchanged' if same else 'changed'}"
    # o: row-wise codes change only in rows 100..131; column-wise codes only in the
    # 32-row blocks holding them (rows 96..159)
    d_q = (synced["o"][0] != synced2["o"][0]).any(dim=1).nonzero().flatten().cpu().numpy()
    assert d_q.size > 0 and d_q.min() >= 100 and d_q.max() <= 131
    d_qt = (synced["o"][2] != synced2["o"][2]).any(dim=0).nonzero().flatten().cpu().numpy()
    assert d_qt.size > 0 and d_qt.min() >= 96 and d_qt.max() <= 159
    # down: one element -> its row block and its column block only
    d_q = (synced["down"][0] != synced2["down"][0]).nonzero().cpu().numpy()
    assert d_q.size > 0 and (d_q[:, 0] == 7).all() and (d_q[:, 1] // 32 == 4000 // 32).all()


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_probe_gemm_every_expert(gpu_lib, which):
    mx = gpu_lib
    _, _, _, w_gu, w_dn = mxsynth.moe_inputs()
    w = w_gu if which == "gate_up" else w_dn
    G, N, K = w.shape
    wflat = w.reshape(G * N, K)
    wq, ws = mx.mx_quantize_rowwise(wflat.cuda())
    owq, ows = oracle_rowwise_par(mxsynth.bits(wflat))
    assert np.array_equal(wq.cpu().numpy(), owq) and np.array_equal(ws.cpu().numpy(), ows)
    # rearranged scales rebuilt per expert from the current quantization
    b_swz = torch.cat([mx.mx_scale_swizzle(ws[g * N:(g + 1) * N]) for g in range(G)])
    # one probe row per expert
    probe = mxsynth.normal_bf16((G, K), 1.0, 77)
    qa, sa = mx.mx_quantize_rowwise(bf16_dev(probe))
    oqa, osa = oracle.quantize_rowwise(mxsynth.bits(probe))
    off = np.arange(G + 1, dtype=np.int64)
    offd = torch.from_numpy(off).cuda()
    C = mx.mx_grouped_gemm(offd, qa, mx.mx_scale_swizzle(sa), wq.view(G, N, K), b_swz,
                           out_dtype=torch.bfloat16)
    ref = grouped_ref(off, oqa, osa, owq.reshape(G, N, K), ows.reshape(G, N, K // 32))
    assert_gemm_close(C, ref, f"probe {which}, all {G} experts x {N} columns")

    # a stale rearranged scale copy of expert 97 (taken before its weights were
    # doubled): its probe row fails, every other row is unchanged
    per = mx.mx_scale_swizzled_bytes(N, K // 32)
    w97 = (wflat[97 * N:98 * N].float() * 2.0).to(torch.bfloat16).cuda()
    wq2 = wq.clone()
    wq2[97 * N:98 * N], s97 = mx.mx_quantize_rowwise(w97)
    C2 = mx.mx_grouped_gemm(offd, qa, mx.mx_scale_swizzle(sa), wq2.view(G, N, K), b_swz,
                            out_dtype=torch.bfloat16)
    fresh = b_swz.clone()
    fresh[97 * per:98 * per] = mx.mx_scale_swizzle(s97)
    C3 = mx.mx_grouped_gemm(offd, qa, mx.mx_scale_swizzle(sa), wq2.view(G, N, K), fresh,
                            out_dtype=torch.bfloat16)
    rows_differ = (C2 != C3).any(dim=1).nonzero().flatten().cpu().tolist()
    assert rows_differ == [97], rows_differ
    # with the stale copy the row is off by the scale step (the codes encode 2w
    # against the old exponents): about half of the fresh result
    r = (C2[97].float() / C3[97].float())[C3[97].float().abs() > 1e-3]
    assert r.numel() > 0 and (r - 0.5).abs().max().item() < 0.02
