"""One full-size step of bench.py, in the launch configuration it times,
checked against the oracle.

bench.py's step fuses several quantizations into single launches (the
layer's seven weights in one dual pass, written into stacked and
side-by-side operands; activations with their scales rearranged in the same
pass; all 128 experts of a stacked weight in one launch; the MoE output
gradients quantized both ways from one read).  This test runs that step once
on its seeded device inputs and compares every quantized output with the
oracle applied to the same input bytes (bit for bit), and lattices of each
kind of GEMM output (an entry in every 256 x 256 tile, every expert's tiles
for the grouped products) at the stated bar against the run-window model of
tests/gpu_util.py.  Outputs computed from other GPU
outputs (the SwiGLU of the gate_up product and what follows it) are covered
by their own tests, since the oracle takes no input from the GPU path."""
import numpy as np
import pytest
import torch

import bench
import mxsynth
import oracle
from gpu_util import (_pool_map, check_sampled, check_sampled_grouped, check_sampled_wgrad,
                      lattice_entries, lattice_grouped, lattice_wgrad, oracle_colwise_par,
                      oracle_rowwise_par)

pytestmark = pytest.mark.gpu


def _eq(got: torch.Tensor, ref: np.ndarray, what: str):
    g = got.cpu().numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    bad = np.argwhere(g != ref)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first at {tuple(bad[0])}"


def _row(mx_q, mx_swz, xbits, what):
    oq, os_ = oracle_rowwise_par(xbits)
    _eq(mx_q, oq, what + " row-wise codes")
    _eq(mx_swz, oracle.scale_swizzle(os_), what + " row-wise scales")
    return oq, os_


def _col(mx_qt, mx_swz, xbits, what):
    oqt, ost = oracle_colwise_par(xbits)
    _eq(mx_qt, oqt, what + " column-wise codes")
    _eq(mx_swz, oracle.scale_swizzle(ost), what + " column-wise scales")
    return oqt, ost


def _experts(w, q, s_swz, qt, st_swz, what):
    """Stacked experts, both orientations; returns the oracle's column-wise stacks."""
    G, N, K = w.shape
    wb = mxsynth.bits(w)
    parts = _pool_map(lambda g: (oracle.quantize_rowwise(wb[g]), oracle.quantize_colwise(wb[g])), range(G))
    _eq(q, np.stack([p[0][0] for p in parts]), what + " row-wise codes")
    _eq(s_swz, np.concatenate([oracle.scale_swizzle(p[0][1]) for p in parts]), what + " row-wise scales")
    _eq(qt, np.stack([p[1][0] for p in parts]), what + " column-wise codes")
    _eq(st_swz, np.concatenate([oracle.scale_swizzle(p[1][1]) for p in parts]), what + " column-wise scales")
    return np.stack([p[1][0] for p in parts]), np.stack([p[1][1] for p in parts])


def _grouped_col(qt, st_swz, pad, xbits, off, k_cap, what):
    parts = _pool_map(lambda c0: oracle.quantize_colwise_grouped(
        np.ascontiguousarray(xbits[:, c0:c0 + 256]), off, k_cap), range(0, xbits.shape[1], 256))
    oqt = np.concatenate([p[0] for p in parts])
    ost = np.concatenate([p[1] for p in parts])
    opad = parts[0][2]
    _eq(pad, opad, what + " ranges")
    pend = int(opad[-1])
    _eq(qt[:, :pend], oqt[:, :pend], what + " per-expert column-wise codes")
    KT = k_cap // 256
    got = st_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256]
    want = oracle.scale_swizzle(ost).reshape(-1, KT, 256)[:, :pend // 256]
    assert np.array_equal(got, want), what + " per-expert column-wise scales"
    return oqt, ost, opad


def test_bench_step_matches_oracle(gpu_lib):
    mx = gpu_lib
    I, o = bench.build_workload(mx, torch, mxsynth)
    bench.step(mx, I, o, lambda cat, fn, *a, **kw: fn(*a, **kw))
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    W = I["W"]
    bits = mxsynth.bits
    print("weight sync", flush=True)
    oqkv = _row(o["qkv_q"], o["qkv_swz"], bits(torch.cat([W["q"], W["k"], W["v"]])), "qkv")
    gu = bits(torch.cat([W["gate"], W["up"]]))
    _row(o["gu_q"], o["gu_swz"], gu, "gate_up")
    oguT = _col(o["guT_q"], o["guT_swz"], gu, "gate_up")
    del gu
    _row(o["o_q"], o["o_swz"], bits(W["o"]), "o")
    _row(o["dn_q"], o["dn_swz"], bits(W["down"]), "down")
    for n in ("q", "k", "v", "o", "down"):
        _col(o["colT"][n], o["colT_swz"][n], bits(W[n]), n)
    print("activations", flush=True)
    oxh = _row(o["xh_q"], o["xh_swz"], bits(I["xh"]), "X (hidden)")
    _row(o["xi_q"], o["xi_swz"], bits(I["xi"]), "X (intermediate)")
    rows, cols = lattice_entries(rng, 4608, 6144)
    check_sampled(o["C_qkv"], rows, cols, oxh[0], oxh[1], oqkv[0], oqkv[1], "qkv product")
    del oxh, oqkv
    print("dense backward", flush=True)
    dyb = bits(I["dy"])
    ody = _row(o["dy_q"], o["dy_swz"], dyb, "dY")
    _col(o["dyT_q"], o["dyT_swz"], dyb, "dY")
    del dyb
    oxT, oxTs = oracle_colwise_par(bits(I["x"]))
    _eq(o["xT_q"], oxT, "X column-wise codes")
    _eq(o["xT_swz"], oracle.scale_swizzle(oxTs), "X column-wise scales")
    rows, cols = lattice_entries(rng, 12288, 4096)
    check_sampled(o["C_dgrad"], rows, cols, ody[0], ody[1], oguT[0], oguT[1], "dgrad product")
    del ody, oguT, oxT, oxTs
    print("MoE forward", flush=True)
    G = I["w_gu"].shape[0]
    ogu_qt, ogu_st = _experts(I["w_gu"], o["mgu_wq"], o["mgu_wswz"], o["mgu_wqt"], o["mgu_wstswz"], "W_gu")
    _experts(I["w_dn"], o["mdn_wq"], o["mdn_wswz"], o["mdn_wqt"], o["mdn_wstswz"], "W_dn")
    ids = I["ids"].cpu().numpy()
    off, src, slot = oracle.moe_dispatch(ids, G)
    _eq(o["moff"], off, "dispatch offsets")
    _eq(o["msrc"], src, "dispatch source tokens")
    _eq(o["mslot"], slot, "dispatch slots")
    _row(o["xq"], o["xswz"], bits(I["x_tok"])[src], "dispatched rows")
    src_rows, M_rows = src, ids.size
    print("MoE backward", flush=True)
    off = I["off"].cpu().numpy()          # the same expert sizes as the routing
    k_cap = I["k_cap"]
    dyb = bits(I["dy_gu"])
    odq = _row(o["mgu_dyq"], o["mgu_dyswz"], dyb, "dY_gu")
    oa = _grouped_col(o["mgu_dyT"], o["mgu_dyTswz"], o["mgu_pad"], dyb, off, k_cap, "dY_gu")
    del dyb
    # data gradient of gate_up: every tile of every expert, and each expert's
    # first and last row
    nz = np.diff(off) > 0
    rl, cl = lattice_grouped(rng, off, 2048)
    r = np.concatenate([rl, off[:-1][nz], off[1:][nz] - 1])
    c = np.concatenate([cl, rng.integers(0, 2048, r.size - rl.size)])
    check_sampled_grouped(o["dX_mgu"], r, c, off, odq[0], odq[1], ogu_qt, ogu_st, "MoE gate_up dgrad")
    del odq, ogu_qt, ogu_st
    # gate_up's weight-gradient operand: the dispatched rows, quantized per
    # expert column-wise by the dispatch itself
    routed = int(off[-1])
    xg = np.zeros((M_rows, 2048), np.uint16)
    xg[:routed] = bits(I["x_tok"])[src_rows[:routed]]
    ob = _grouped_col(o["mgu_xT"], o["mgu_xTswz"], o["mgu_pad2"], xg, off, k_cap, "X_gu")
    del xg
    # weight gradient of gate_up: every 256 x 256 tile of every expert
    gs, rs, cs = lattice_wgrad(rng, G, 1536, 2048)
    check_sampled_wgrad(o["dW_mgu"], gs, rs, cs, oa[2], oa[0], oa[1], ob[0], ob[1], "MoE gate_up wgrad")
