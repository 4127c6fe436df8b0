"""mx_moe_dispatch_noalloc (chunk counts in the library's device array)
against mx_moe_dispatch (chunk counts in a caller's workspace), through the
C ABI: every output byte equal, on consecutive calls of different sizes --
the largest routing the array holds (262 144 assignments over 1024
experts), then smaller ones -- so that a call's counts never leak into the
next.  The routing index work is also checked against the oracle's stable
sort by expert."""
import numpy as np
import pytest
import torch

import mxsynth
import oracle

pytestmark = pytest.mark.gpu


def _routing(rng, T, k, E):
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)   # k distinct experts
    return ids


def _both(mx, x, ids_np, E):
    T, k = ids_np.shape
    n = T * k
    H = x.shape[1]
    dev = "cuda"
    ids = torch.from_numpy(ids_np).to(dev)
    outs = []
    for fn in ("ws", "noalloc"):
        off = torch.full((E + 1,), -7, dtype=torch.int64, device=dev)
        src = torch.full((n,), -7, dtype=torch.int32, device=dev)
        slot = torch.full((n,), -7, dtype=torch.int32, device=dev)
        q = torch.full((n, H), 0x55, dtype=torch.uint8, device=dev)
        s = torch.full((mx.mx_scale_swizzled_bytes(n, H // 32),), 0x55, dtype=torch.uint8, device=dev)
        if fn == "ws":
            mx.mx_moe_dispatch(x, ids, E, offsets=off, src=src, slot=slot, q=q, s_swz=s)
        else:
            mx.mx_moe_dispatch_noalloc(x, ids, E, off, src, slot, q, s)
        torch.cuda.synchronize()
        outs.append((off, src, slot, q, s))
    return outs


def test_noalloc_matches_workspace_dispatch(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(123)
    # the largest routing the 4 MiB array holds, then smaller ones
    for T, k, E, H in ((32768, 8, 1024, 256), (2048, 8, 128, 512), (300, 4, 16, 256)):
        print(f"noalloc dispatch T={T} top-{k} E={E} H={H}", flush=True)
        assert mx.mx_moe_dispatch_workspace_bytes(T, k, E) <= 4 << 20
        x = mxsynth.normal_bf16((T, H), 1.0, seed=T + E).cuda()
        ids = _routing(rng, T, k, E)
        (o1, s1, l1, q1, w1), (o2, s2, l2, q2, w2) = _both(mx, x, ids, E)
        assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(l1, l2)
        assert torch.equal(q1, q2) and torch.equal(w1, w2)
        off, src, slot = oracle.moe_dispatch(ids, E)
        assert np.array_equal(o2.cpu().numpy(), off)
        assert np.array_equal(s2.cpu().numpy(), src)
        assert np.array_equal(l2.cpu().numpy(), slot)


def test_noalloc_refuses_beyond_its_array(gpu_lib):
    mx = gpu_lib
    T, k, E, H = 32800, 8, 1024, 256
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    n = T * k
    args = [torch.empty(E + 1, dtype=torch.int64, device="cuda"), torch.empty(n, dtype=torch.int32, device="cuda"),
            torch.empty(n, dtype=torch.int32, device="cuda"), torch.empty((n, H), dtype=torch.uint8, device="cuda"),
            torch.empty(mx.mx_scale_swizzled_bytes(n, H // 32), dtype=torch.uint8, device="cuda")]
    with pytest.raises(mx.MxError) as e:
        mx.mx_moe_dispatch_noalloc(x, ids, E, *args)
    assert e.value.status == mx.MX_ERR_UNSUPPORTED
