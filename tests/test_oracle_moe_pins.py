"""Pins of the oracle's MoE dispatch order and combine (CPU).

The dispatch order is defined as a stable sort of the routed assignments by
expert; the pins rebuild it with the plainest possible loop (walk the experts
in order, and for each the assignments in order) and check the invariants a
plausible mistake would break (offsets, inverse maps, stability, unrouted
ids).  The combine is pinned by special cases with exact answers."""
import numpy as np

import oracle


def _loop_order(ids, G):
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    rows = []
    for e in range(G):
        for a in range(flat.size):
            if flat[a] == e:
                rows.append(a)
    return rows


def test_dispatch_equals_loop_definition():
    rng = np.random.default_rng(1)
    for T, k, G in ((1, 1, 1), (5, 3, 4), (17, 2, 7), (40, 8, 16)):
        ids = rng.integers(-1, G + 1, size=(T, k))          # includes unrouted -1 and G
        off, src, slot = oracle.moe_dispatch(ids, G)
        rows = _loop_order(ids, G)
        assert off[-1] == len(rows)
        for i, a in enumerate(rows):
            assert src[i] == a // k and slot[a] == i
        assert (src[len(rows):] == -1).all()
        flat = ids.reshape(-1)
        assert ((slot == -1) == ((flat < 0) | (flat >= G))).all()
        for e in range(G):
            assert off[e + 1] - off[e] == int((flat == e).sum())


def test_dispatch_invariants_large():
    rng = np.random.default_rng(2)
    T, k, G = 3000, 8, 128
    p = 1.0 / np.arange(1, G + 1) ** 1.1
    ids = np.stack([rng.choice(G, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    off, src, slot = oracle.moe_dispatch(ids, G)
    n = T * k
    assert off[0] == 0 and off[-1] == n and (np.diff(off) >= 0).all()
    assert sorted(slot.tolist()) == list(range(n))          # a bijection onto the rows
    flat = ids.reshape(-1)
    assert (src[slot] == np.arange(n) // k).all()
    for e in (0, 5, 127):
        a = np.nonzero(flat == e)[0]
        assert (slot[a] == np.arange(off[e], off[e + 1])).all()  # stable: in assignment order


def test_combine_special_cases():
    rng = np.random.default_rng(3)
    T, k, H = 6, 3, 16
    n = T * k
    y = rng.integers(-50, 50, size=(n, H)).astype(np.float32)
    ybits = (y.view(np.uint32) >> 16).astype(np.uint16)   # small integers: exact in BF16
    slot = rng.permutation(n).astype(np.int32)
    # one-hot weights: a gather
    w = np.zeros((T, k), np.float32)
    w[:, 1] = 1.0
    out, bnd = oracle.moe_combine(ybits, slot, w)
    assert np.array_equal(out, y[slot.reshape(T, k)[:, 1]].astype(np.float64))
    # weights 1, 2, 4: exact integer sums
    w = np.tile(np.array([1.0, 2.0, 4.0], np.float32), (T, 1))
    out, _ = oracle.moe_combine(ybits, slot, w)
    s = slot.reshape(T, k)
    assert np.array_equal(out, y[s[:, 0]] + 2 * y[s[:, 1]] + 4 * y[s[:, 2]])
    # an unrouted slot contributes nothing
    s2 = slot.copy()
    s2[0] = -1
    out2, _ = oracle.moe_combine(ybits, s2, w)
    assert np.array_equal(out2[0], 2 * y[s[0, 1]] + 4 * y[s[0, 2]])
    assert np.array_equal(out2[1:], out[1:])
