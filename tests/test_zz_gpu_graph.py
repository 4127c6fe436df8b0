"""HIP graph capture of the library's calls (the MoE layer pass at small sizes).

One pass -- dual quantization of stacked expert weights, dispatch, grouped
gate_up, SwiGLU + quantize, grouped down, combine, row-wise quantization with
rearranged scales, per-expert column-wise quantization and the weight
gradient, plus a dense GEMM with a split tail -- is run eagerly, then captured
into a graph on the same stream and replayed three times with eager work and
synchronizations between the replays.  Every output is deterministic, so
every replay must reproduce the eager bytes exactly.  The calls that need
scratch memory take one caller-owned workspace; the library holds no state,
so a graph whose capture holds the very first calls of the process's stream
(test_first_calls_inside_capture) replays as exactly.
"""
import numpy as np
import pytest
import torch

import mxsynth

pytestmark = pytest.mark.gpu


def _pass(mx, I, o):
    mx.mx_quantize_dual_experts(I["w_gu"], q=o["wgu_q"], s_swz=o["wgu_s"], qt=o["wgu_qt"], st_swz=o["wgu_st"])
    mx.mx_quantize_dual_experts(I["w_dn"], q=o["wdn_q"], s_swz=o["wdn_s"], qt=o["wdn_qt"], st_swz=o["wdn_st"])
    mx.mx_moe_dispatch(I["x"], I["ids"], I["G"], offsets=o["off"], src=o["src"], slot=o["slot"],
                       q=o["xq"], s_swz=o["xs"], workspace=I["ws"])
    mx.mx_grouped_gemm(o["off"], o["xq"], o["xs"], o["wgu_q"], o["wgu_s"], c=o["gu"])
    mx.mx_swiglu_quantize(o["gu"], q=o["hq"], s_swz=o["hs"], h=o["h"])
    mx.mx_grouped_gemm(o["off"], o["hq"], o["hs"], o["wdn_q"], o["wdn_s"], c=o["dn"])
    mx.mx_moe_combine(o["dn"], o["slot"], I["w"], out=o["out"])
    mx.mx_quantize_rowwise_swz(I["dy"], q=o["dyq"], s_swz=o["dys"])
    mx.mx_grouped_gemm(o["off"], o["dyq"], o["dys"], o["wdn_qt"], o["wdn_st"], c=o["dh"])
    mx.mx_quantize_colwise_grouped(I["dy"], o["off"], k_cap=I["k_cap"], qt=o["dyT"], st_swz=o["dyTs"],
                                   pad_offsets=o["pad"])
    mx.mx_quantize_colwise_grouped(o["h"], o["off"], k_cap=I["k_cap"], qt=o["hT"], st_swz=o["hTs"],
                                   pad_offsets=o["pad2"])
    mx.mx_grouped_gemm_wgrad(o["pad"], o["dyT"], o["dyTs"], o["hT"], o["hTs"], c=o["dw"], workspace=I["ws"])
    # a dense product whose tile count leaves a partial round: split tail
    mx.mx_gemm(o["dyq"][:1280], o["dys"], o["wgu_qt"][0], o["wgu_st"], c=o["dense"], workspace=I["ws"])


def _setup(mx, dev="cuda"):
    """Inputs I (with the shared workspace I["ws"]) and output buffers o."""
    T, H, F, G, k = 640, 512, 256, 8, 4
    rng = np.random.default_rng(9)
    ids = np.stack([rng.choice(G, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    I = dict(x=mxsynth.normal_bf16((T, H), 1.0, seed=1).to(dev),
             ids=torch.from_numpy(ids).to(dev), w=torch.from_numpy(w / w.sum(1, keepdims=True)).to(dev),
             w_gu=mxsynth.normal_bf16((G, 2 * F, H), 0.02, seed=2).to(dev),
             w_dn=mxsynth.normal_bf16((G, H, F), 0.02, seed=3).to(dev),
             dy=mxsynth.normal_bf16((T * k, H), 1e-3, seed=4).to(dev), G=G)
    n = T * k
    I["k_cap"] = mx.mx_grouped_k_capacity(n, G)
    u8 = dict(dtype=torch.uint8, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    swz = mx.mx_scale_swizzled_bytes
    o = dict(wgu_q=torch.empty(G, 2 * F, H, **u8), wgu_s=torch.empty(G * swz(2 * F, H // 32), **u8),
             wgu_qt=torch.empty(G, H, 2 * F, **u8), wgu_st=torch.empty(G * swz(H, 2 * F // 32), **u8),
             wdn_q=torch.empty(G, H, F, **u8), wdn_s=torch.empty(G * swz(H, F // 32), **u8),
             wdn_qt=torch.empty(G, F, H, **u8), wdn_st=torch.empty(G * swz(F, H // 32), **u8),
             off=torch.empty(G + 1, dtype=torch.int64, device=dev),
             src=torch.empty(n, dtype=torch.int32, device=dev), slot=torch.empty(n, dtype=torch.int32, device=dev),
             xq=torch.empty(n, H, **u8), xs=torch.empty(swz(n, H // 32), **u8),
             gu=torch.empty(n, 2 * F, **bf), hq=torch.empty(n, F, **u8), hs=torch.empty(swz(n, F // 32), **u8),
             h=torch.empty(n, F, **bf), dn=torch.empty(n, H, **bf), out=torch.empty(T, H, **bf),
             dyq=torch.empty(n, H, **u8), dys=torch.empty(swz(n, H // 32), **u8), dh=torch.empty(n, F, **bf),
             dyT=torch.empty(H, I["k_cap"], **u8), dyTs=torch.empty(swz(H, I["k_cap"] // 32), **u8),
             hT=torch.empty(F, I["k_cap"], **u8), hTs=torch.empty(swz(F, I["k_cap"] // 32), **u8),
             pad=torch.empty(G + 1, dtype=torch.int64, device=dev),
             pad2=torch.empty(G + 1, dtype=torch.int64, device=dev),
             dw=torch.empty(G, H, F, **bf), dense=torch.empty(1280, H, **bf))
    assert mx.mx_gemm_workspace_bytes(1280, H, 2 * F) > 0, "the dense product must take the split tail"
    I["ws"] = torch.empty(max(mx.mx_gemm_workspace_bytes(1280, H, 2 * F), mx.mx_moe_dispatch_workspace_bytes(T, k, G),
                              mx.mx_grouped_gemm_wgrad_workspace_bytes()), **u8)
    return I, o


def _written(I, o, k_):
    """Only the bytes each call defines: the codes past pad[G] and the GEMM
    rows of unrouted assignments are not written by design."""
    t = o[k_]
    pend = int(o["pad"][-1])
    if k_ in ("dyT", "hT"):
        return t[:, :pend]
    if k_ in ("dyTs", "hTs"):                     # [32-row tiles][k_cap/256 tiles][256]
        return t.view(-1, I["k_cap"] // 256, 256)[:, :pend // 256]
    return t


def _replay_and_compare(g, I, o, ref):
    keys = list(o)
    for rep in range(3):
        for k_ in keys:                     # eager work between replays: clobber the outputs
            o[k_].view(torch.uint8).fill_(0xA5)
        I["ws"].fill_(0x5A)                 # and the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k_ in keys:
            assert torch.equal(_written(I, o, k_).contiguous().view(torch.uint8),
                               ref[k_].contiguous().view(torch.uint8)), f"replay {rep}: {k_} differs"


def test_graph_replays_match_eager(gpu_lib):
    mx = gpu_lib
    I, o = _setup(mx)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _pass(mx, I, o)                     # eager
    torch.cuda.synchronize()
    ref = {k_: _written(I, o, k_).clone() for k_ in o}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _pass(mx, I, o)
    _replay_and_compare(g, I, o, ref)


def test_first_calls_inside_capture(gpu_lib):
    """A fresh stream whose first library calls are made inside capture; the
    eager reference runs afterwards on another stream with its own buffers."""
    mx = gpu_lib
    I, o = _setup(mx)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _pass(mx, I, o)
    I2, o2 = _setup(mx)
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        _pass(mx, I2, o2)
    torch.cuda.synchronize()
    ref = {k_: _written(I2, o2, k_).clone() for k_ in o2}
    _replay_and_compare(g, I, o, ref)
