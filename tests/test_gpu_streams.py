"""Calls on different streams: a split-tail GEMM, a MoE dispatch and a
weight gradient issued on two streams at once, each call with its own
workspace (the binding takes one from torch's allocator for the current
stream when none is passed), give the same bytes as the same calls on one
stream.  The result of every call is deterministic, so the comparison is
exact."""
import numpy as np
import pytest
import torch

import mxsynth
from gpu_util import random_mx_operand, to_dev

pytestmark = pytest.mark.gpu


def _work(mx, I, c_gemm, d_out, w_out):
    # 4608 x 4096 x 4096: 288 tiles, the partial last round split along K
    mx.mx_gemm(I["a"], I["as"], I["b"], I["bs"], c=c_gemm)
    off, src, slot, q, s = mx.mx_moe_dispatch(I["x"], I["ids"], 16)
    d_out.copy_(q[:, :64])
    qa, sa, pad = mx.mx_quantize_colwise_grouped(I["dy"], off)
    qb, sb, _ = mx.mx_quantize_colwise_grouped(I["h"], off)
    mx.mx_grouped_gemm_wgrad(pad, qa, sa, qb, sb, c=w_out)


def test_two_streams_match_one(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(17)
    qa, sa = random_mx_operand(rng, 4608, 4096)
    qb, sb = random_mx_operand(rng, 4096, 4096)
    T, k, G = 1024, 4, 16
    ids = np.stack([rng.choice(G, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    n = T * k
    I = dict(a=to_dev(qa), as_=None, b=to_dev(qb),
             x=mxsynth.normal_bf16((T, 256), 1.0, seed=31).cuda(), ids=torch.from_numpy(ids).cuda(),
             dy=mxsynth.normal_bf16((n, 256), 1e-3, seed=32).cuda(),
             h=mxsynth.normal_bf16((n, 256), 1.0, seed=33).cuda())
    I["as"] = mx.mx_scale_swizzle(to_dev(sa))
    I["bs"] = mx.mx_scale_swizzle(to_dev(sb))
    mk = lambda: (torch.empty(4608, 4096, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(n, 64, dtype=torch.uint8, device="cuda"),
                  torch.empty(G, 256, 256, dtype=torch.bfloat16, device="cuda"))
    ref = mk()
    _work(mx, I, *ref)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [mk(), mk()]
    for rep in range(2):
        for s, o in zip((s1, s2), outs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                _work(mx, I, *o)
        torch.cuda.synchronize()
        for o in outs:
            for got, want in zip(o, ref):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
