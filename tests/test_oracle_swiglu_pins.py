"""Pins of the oracle's SwiGLU between the MoE expert projections (CPU).

h = silu(g) * u with silu(g) = g / (1 + exp(-g)) (Qwen3's expert MLP; paper
Table 2), rounded once to BF16 (activations are BF16, paper Figure 1) and then
quantized row-wise (the quantizer has its own pins).

  - the double -> BF16 rounding against a brute-force nearest search over
    every finite BF16 value (ties to the even pattern), and the identity on
    every BF16 value;
  - silu against closed forms: silu(g) - silu(-g) = g, sigma(ln 3) = 3/4,
    silu(0) = 0, silu(g) = g once exp(-g) is below half a double ulp, and
    linearity in u;
  - the array routine's layout (gate columns first, up columns second)."""
import math

import numpy as np

import oracle


def _all_bf16():
    """Every finite BF16 pattern and its exact value."""
    pat = np.arange(65536, dtype=np.uint32)
    f = (pat << 16).view(np.float32)
    ok = np.isfinite(f)
    val = np.where(ok, f, 0).astype(np.float64)
    return pat[ok].astype(np.uint16), val[ok]


def _nearest_bf16(v, pats, vals):
    d = np.abs(vals - v)
    best = d.min()
    cands = pats[d == best]
    if cands.size > 1:                        # a tie: the even pattern (or +-0)
        cands = cands[(cands & 1) == 0]
    c = int(cands[0])
    if abs(v) >= 2.0 ** 128 * (1 - 2.0 ** -9):  # rounds past the largest finite
        c = 0x7F80 | (0x8000 if v < 0 else 0)
    return c


def test_double_to_bf16_brute_force():
    pats, vals = _all_bf16()
    # one of each sign of zero: the search above sees +0 and -0 at distance 0
    rng = np.random.default_rng(0)
    xs = []
    for e in rng.integers(-140, 128, size=600):
        xs.append(float(rng.uniform(1, 2) * 2.0 ** int(e)) * (1 if rng.random() < 0.5 else -1))
    # exact midpoints between neighbours (ties) and points next to them
    for i in rng.integers(0, vals.size - 1, size=300):
        a, b = vals[i], vals[i + 1]
        if np.isfinite(a) and np.isfinite(b) and np.sign(a) == np.sign(b) and a != 0 and b != 0:
            m = (a + b) / 2
            xs += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf)]
    for x in xs:
        want = _nearest_bf16(x, pats, vals)
        got = oracle.double_to_bf16(x)
        if want in (0x0000, 0x8000):           # zero: keep the sign of x
            want = 0x8000 if x < 0 else 0x0000
        assert got == want, (x, hex(got), hex(want))


def test_double_to_bf16_identity_on_bf16_values():
    pats, vals = _all_bf16()
    for p, v in zip(pats[::7], vals[::7]):
        assert oracle.double_to_bf16(float(v)) == int(p)
    assert oracle.double_to_bf16(float("inf")) == 0x7F80
    assert oracle.double_to_bf16(-float("inf")) == 0xFF80
    assert oracle.double_to_bf16(2.0 ** 128) == 0x7F80
    assert oracle.double_to_bf16(-0.0) == 0x8000


def test_silu_closed_forms():
    rng = np.random.default_rng(1)
    for g in rng.normal(0, 4, size=200):
        g = float(g)
        d = oracle.swiglu_f64(g, 1.0) - oracle.swiglu_f64(-g, 1.0)
        assert abs(d - g) <= 4e-16 * max(1.0, abs(g))
        u = float(rng.normal())
        assert oracle.swiglu_f64(g, 2 * u) == 2 * oracle.swiglu_f64(g, u)
    ln3 = math.log(3.0)
    assert abs(oracle.swiglu_f64(ln3, 1.0) - 0.75 * ln3) <= 2e-16
    assert oracle.swiglu_f64(0.0, 5.0) == 0.0
    for g in (40.0, 64.0, 1000.0):
        assert oracle.swiglu_f64(g, 3.0) == 3.0 * g
    assert oracle.swiglu_f64(-1000.0, 3.0) == 0.0 or abs(oracle.swiglu_f64(-1000.0, 3.0)) < 1e-300


def test_swiglu_array_layout():
    # gate 64 (silu(64) = 64 exactly): h = 64 u, exact in BF16 for BF16 u;
    # with the halves swapped it would be silu(u) * 64
    rows, F = 3, 40
    u = np.linspace(-3, 3, rows * F).astype(np.float32).reshape(rows, F)
    u_bits = (u.view(np.uint32) >> 16).astype(np.uint16)
    u = (u_bits.astype(np.uint32) << 16).view(np.float32)
    g_bits = np.full((rows, F), 0x4280, np.uint16)          # 64.0
    h = oracle.swiglu_bf16(np.concatenate([g_bits, u_bits], axis=1))
    want = ((64.0 * u).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(h, want)
    # zero gate: zero output (+0 for u >= 0, -0 for u < 0 is a sign detail
    # the test does not pin; compare values)
    h0 = oracle.swiglu_bf16(np.concatenate([np.zeros((rows, F), np.uint16), u_bits], axis=1))
    assert ((h0.astype(np.uint32) << 16).view(np.float32) == 0).all()
