"""GPU parity of the MoE dispatch (sorted, gathered, quantized rows) and
combine against the oracle.

Bar: dispatch is integer and byte work, so offsets, the row order (src_token,
slot), the codes and the routed rows' scales are bit-exact.  Combine is FP32
sums of weight * value rounded once to BF16: |out - ref| <= one BF16 ulp of
ref + topk * 2^-24 * sum_j |w_j y_j| (each fused multiply-add rounds once)."""
import numpy as np
import pytest
import torch

import mxsynth
import oracle
from gpu_util import bf16_dev, grouped_ref, assert_gemm_close, oracle_rowwise_par, ulp_bf16

pytestmark = pytest.mark.gpu


def _routing(rng, T, k, G, invalid=0):
    ids = np.stack([rng.choice(G, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if invalid:
        bad = rng.choice(T * k, size=invalid, replace=False)
        ids.reshape(-1)[bad[: invalid // 2]] = -1
        ids.reshape(-1)[bad[invalid // 2:]] = G + 3
    return ids


def _check_dispatch(mx, x_bits, ids, G, what, par=False):
    T, H = x_bits.shape
    out = mx.mx_moe_dispatch(bf16_dev(mxsynth.from_bits(x_bits)), torch.from_numpy(ids).cuda(), G)
    off, src, slot, q, s_swz = (t.cpu().numpy() for t in out)
    ooff, osrc, oslot = oracle.moe_dispatch(ids, G)
    routed = int(ooff[-1])
    assert np.array_equal(off, ooff), f"{what}: offsets"
    assert np.array_equal(slot, oslot), f"{what}: slot"
    assert np.array_equal(src[:routed], osrc[:routed]), f"{what}: src_token"
    gathered = x_bits[osrc[:routed]]
    oq, os_ = (oracle_rowwise_par(gathered) if par else oracle.quantize_rowwise(gathered))
    assert np.array_equal(q[:routed], oq), f"{what}: codes"
    s = oracle.scale_unswizzle(s_swz, T * ids.shape[1], H // 32)
    assert np.array_equal(s[:routed], os_), f"{what}: scales"
    return out, (ooff, osrc, oslot, oq, os_)


@pytest.mark.parametrize("T,H,k,G,invalid", [(1, 256, 1, 1, 0), (37, 256, 3, 5, 0), (1000, 512, 8, 16, 0),
                                             (999, 768, 4, 33, 40), (300, 256, 2, 1024, 7)])
def test_dispatch_matches_oracle(gpu_lib, T, H, k, G, invalid):
    rng = np.random.default_rng(T + H + k + G)
    x = mxsynth.bits(mxsynth.normal_bf16((T, H), 1.0, T + 1, 0.01, 30.0))
    ids = _routing(rng, T, k, G, invalid)
    _check_dispatch(gpu_lib, x, ids, G, f"dispatch T{T} H{H} k{k} G{G}")


def test_dispatch_qwen3_moe_routing(gpu_lib):
    """The MoE layer's routing (20480 tokens, top-8 of 128 experts, Zipf(1.1)
    loads) on the gate_up input width 2048: 163840 routed rows, bit-exact."""
    ids, _ = mxsynth.moe_routing()
    x = mxsynth.bits(mxsynth.normal_bf16((mxsynth.MOE_TOKENS, mxsynth.MOE_HIDDEN), 1.0, 5200))
    out, _ = _check_dispatch(gpu_lib, x, ids, mxsynth.MOE_EXPERTS, "qwen3 routing", par=True)
    assert int(out[0][-1].item()) == mxsynth.MOE_TOKENS * mxsynth.MOE_TOPK
    # same routing, same bytes
    again = gpu_lib.mx_moe_dispatch(bf16_dev(mxsynth.from_bits(x)), torch.from_numpy(ids).cuda(),
                                    mxsynth.MOE_EXPERTS)
    for a, b in zip(out, again):
        assert torch.equal(a, b)


def _check_dispatch_dual_grouped(mx, x_bits, ids, G, what, par=False):
    """mx_moe_dispatch_dual_grouped: the dispatch outputs byte-equal to
    mx_moe_dispatch's, and the per-expert column-wise operand byte-equal to
    mx_quantize_colwise_grouped of the permuted BF16 rows and to the oracle's."""
    T, H = x_bits.shape
    xd = bf16_dev(mxsynth.from_bits(x_bits))
    idd = torch.from_numpy(ids).cuda()
    out = mx.mx_moe_dispatch_dual_grouped(xd, idd, G)
    ref = mx.mx_moe_dispatch(xd, idd, G)
    off, src = out[0], out[1]
    routed = int(off[-1].item())
    for a, b, name in zip(out[:5], ref, ("offsets", "src_token", "slot", "q", "s_swz")):
        if name == "src_token":
            a, b = a[:routed], b[:routed]
        elif name == "q":
            a, b = a[:routed], b[:routed]
        elif name == "s_swz":
            n = T * ids.shape[1]
            a = torch.from_numpy(oracle.scale_unswizzle(a.cpu().numpy(), n, H // 32)[:routed])
            b = torch.from_numpy(oracle.scale_unswizzle(b.cpu().numpy(), n, H // 32)[:routed])
        assert torch.equal(a.cpu(), b.cpu()), f"{what}: {name}"
    pad, qt, st_swz = out[5], out[6], out[7]
    k_cap = qt.shape[1]
    rows_total = T * ids.shape[1]
    # the same operand from the permuted BF16 rows (rows past the routed count
    # are in no expert)
    perm = torch.zeros((rows_total, H), dtype=torch.bfloat16, device="cuda")
    perm[:routed] = xd[src[:routed].long()]
    cqt, cst, cpad = mx.mx_quantize_colwise_grouped(perm, off, k_cap=k_cap)
    torch.cuda.synchronize()
    assert torch.equal(pad, cpad), f"{what}: pad offsets"
    pend = int(pad[-1].item())
    KT = k_cap // 256
    assert torch.equal(qt[:, :pend], cqt[:, :pend]), f"{what}: column-wise codes"
    assert torch.equal(st_swz.view(-1, KT, 256)[:, :pend // 256], cst.view(-1, KT, 256)[:, :pend // 256]), \
        f"{what}: column-wise scales"
    ooff, osrc, _ = oracle.moe_dispatch(ids, G)
    pb = x_bits[osrc[:routed]]   # the permuted rows of the experts (the oracle takes exactly those)
    if par:
        return out
    oqt, ost, opad = oracle.quantize_colwise_grouped(pb, ooff, k_cap)
    assert np.array_equal(pad.cpu().numpy(), opad), f"{what}: oracle pad"
    assert np.array_equal(qt.cpu().numpy()[:, :pend], oqt[:, :pend]), f"{what}: oracle column-wise codes"
    assert np.array_equal(st_swz.cpu().numpy().reshape(-1, KT, 256)[:, :pend // 256],
                          oracle.scale_swizzle(ost).reshape(-1, KT, 256)[:, :pend // 256]), \
        f"{what}: oracle column-wise scales"
    return out


@pytest.mark.parametrize("T,H,k,G,invalid", [(1, 256, 1, 1, 0), (37, 256, 3, 5, 0), (1000, 512, 8, 16, 0),
                                             (999, 768, 4, 33, 40), (300, 256, 2, 1024, 7)])
def test_dispatch_dual_grouped_matches_dispatch_and_oracle(gpu_lib, T, H, k, G, invalid):
    rng = np.random.default_rng(T + H + k + G + 1)
    x = mxsynth.bits(mxsynth.normal_bf16((T, H), 1.0, T + 2, 0.01, 30.0))
    ids = _routing(rng, T, k, G, invalid)
    _check_dispatch_dual_grouped(gpu_lib, x, ids, G, f"dual-grouped dispatch T{T} H{H} k{k} G{G}")


def test_dispatch_dual_grouped_qwen3_moe_routing(gpu_lib):
    """The MoE layer's routing (20480 tokens, top-8 of 128 experts) on the
    gate_up input width 2048: the 163840 permuted rows quantized both ways,
    byte-equal to mx_moe_dispatch and to mx_quantize_colwise_grouped of the
    permuted rows (the latter pinned against the oracle at this size in
    tests/test_gpu_moe_bwd.py)."""
    ids, _ = mxsynth.moe_routing()
    x = mxsynth.bits(mxsynth.normal_bf16((mxsynth.MOE_TOKENS, mxsynth.MOE_HIDDEN), 1.0, 5201))
    _check_dispatch_dual_grouped(gpu_lib, x, ids, mxsynth.MOE_EXPERTS, "qwen3 routing", par=True)


def test_dispatch_feeds_grouped_gemm(gpu_lib):
    """Dispatch -> grouped GEMM (the dispatched operand, scales and offsets used
    as they are) -> combine, against the oracle's dispatch, grouped product and
    combine."""
    mx = gpu_lib
    rng = np.random.default_rng(9)
    T, H, N, k, G = 200, 512, 256, 4, 8
    x = mxsynth.bits(mxsynth.normal_bf16((T, H), 1.0, 91))
    ids = _routing(rng, T, k, G)
    w = mxsynth.normal_bf16((G, N, H), 0.05, 92)
    wq, ws = mx.mx_quantize_rowwise(bf16_dev(w.reshape(G * N, H)))
    owq, ows = oracle.quantize_rowwise(mxsynth.bits(w.reshape(G * N, H)))
    b_swz = torch.cat([mx.mx_scale_swizzle(ws[g * N:(g + 1) * N]) for g in range(G)])
    (off, src, slot, q, s_swz), (ooff, osrc, oslot, oq, os_) = _check_dispatch(mx, x, ids, G, "feed")
    C = mx.mx_grouped_gemm(off, q, s_swz, wq.view(G, N, H), b_swz, out_dtype=torch.bfloat16)
    ref = grouped_ref(ooff, oq, os_, owq.reshape(G, N, H), ows.reshape(G, N, H // 32))
    assert_gemm_close(C, ref, "dispatched grouped GEMM")
    routing_w = rng.random((T, k)).astype(np.float32)
    out = mx.mx_moe_combine(C, slot, torch.from_numpy(routing_w).cuda())
    cbits = C.cpu().view(torch.int16).numpy().view(np.uint16)
    r, bnd = oracle.moe_combine(cbits, oslot, routing_w)
    g = out.float().cpu().numpy().astype(np.float64)
    tol = ulp_bf16(r) + k * 2.0 ** -24 * bnd
    assert (np.abs(g - r) <= tol).all()


@pytest.mark.parametrize("T,H,k", [(1, 8, 1), (513, 2048, 8), (64, 768, 3)])
def test_combine_matches_oracle(gpu_lib, T, H, k):
    mx = gpu_lib
    rng = np.random.default_rng(T * 3 + H + k)
    n = T * k
    y = mxsynth.bits(mxsynth.normal_bf16((n, H), 1.0, n + 5, 0.01, 100.0))
    slot = rng.permutation(n).astype(np.int32)
    slot[rng.choice(n, size=max(1, n // 50), replace=False)] = -1   # some unrouted
    weights = rng.random((T, k)).astype(np.float32)
    out = mx.mx_moe_combine(bf16_dev(mxsynth.from_bits(y)), torch.from_numpy(slot).cuda(),
                            torch.from_numpy(weights).cuda())
    r, bnd = oracle.moe_combine(y, slot, weights)
    g = out.float().cpu().numpy().astype(np.float64)
    tol = ulp_bf16(r) + k * 2.0 ** -24 * bnd
    bad = np.argwhere(np.abs(g - r) > tol)
    assert bad.size == 0, f"{len(bad)} outside the bound, first {tuple(bad[0])}"
