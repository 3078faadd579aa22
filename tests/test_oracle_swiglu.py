"""Pins of the oracle's gated feed-forward activation h = silu(g) * u
(model card "Neutrino-1 8B", "Architecture": a gated SwiGLU feed-forward of
three linears per layer) and of the fp32 exp it is evaluated with, against
fp64 mathematics that does not go through the oracle's steps."""
import numpy as np

import oracle


def _ulp(a64, ref64):
    ref32 = ref64.astype(np.float32)
    return np.abs(a64 - ref64) / np.spacing(np.abs(ref32)).astype(np.float64)


def test_exp32_within_ulp_of_exp():
    x = np.linspace(-87.0, 88.7, 1_000_001).astype(np.float32)
    e = oracle.exp32(x).astype(np.float64)
    assert np.all(np.isfinite(e))
    assert _ulp(e, np.exp(x.astype(np.float64))).max() <= 1.5


def test_exp32_special_points():
    e = oracle.exp32(np.array([0.0, 1.0, -1.0, np.log(2.0)], np.float32)).astype(np.float64)
    assert e[0] == 1.0
    assert _ulp(e[1:], np.exp(np.array([1.0, -1.0, np.float32(np.log(2.0))], np.float64))).max() <= 1.0
    # past the largest finite result it overflows to +inf, never to a wrong finite value
    assert np.isinf(oracle.exp32(np.array([89.0, 100.0], np.float32))).all()


def test_swiglu_matches_fp64_definition():
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.normal(0, 3, 20000), rng.uniform(-87, 87, 20000)]).astype(np.float32)
    u = rng.normal(0, 2, g.size).astype(np.float32)
    h = oracle.swiglu(g[None], u[None])[0].astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64)) * u64
    # fp32 steps: exp (<= 1.5 ulp), the sum, the division, the product
    tol = 5 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-37
    assert np.all(np.abs(h - ref) <= tol)


def test_swiglu_closed_forms():
    g = np.array([0.0, 17.0, 30.0, 1e4, -89.0, -1e30], np.float32)
    u = np.array([3.0, -2.5, 0.75, 1.0, 2.0, 5.0], np.float32)
    h = oracle.swiglu(g[None], u[None])[0]
    assert h[0] == 0.0
    # e^-17 < 2^-24: 1 + e rounds to 1, so silu(g) is g and h the fp32 product g * u
    assert np.array_equal(h[1:4], (g[1:4] * u[1:4]).astype(np.float32))
    # very negative gates: silu(g) underflows to -0
    assert np.all(h[4:] == 0.0) and np.all(np.signbit(h[4:]))


def test_swiglu_odd_part_identity():
    # silu(x) - silu(-x) = x (sigma(x) + sigma(-x) = 1), within the fp32 steps' rounding
    x = np.linspace(-40.0, 40.0, 8001).astype(np.float32)
    one = np.ones_like(x)
    d = oracle.swiglu(x[None], one[None])[0].astype(np.float64) - \
        oracle.swiglu((-x)[None], one[None])[0].astype(np.float64)
    assert np.all(np.abs(d - x.astype(np.float64)) <= 4 * np.spacing(np.abs(x)).astype(np.float64) + 1e-30)


def test_swiglu_row_strides_and_tokens():
    rng = np.random.default_rng(3)
    g = rng.normal(0, 2, (5, 300)).astype(np.float32)
    u = rng.normal(0, 2, (5, 300)).astype(np.float32)
    h = oracle.swiglu(g, u)
    for m in range(5):  # rows are independent
        assert np.array_equal(h[m], oracle.swiglu(g[m:m + 1], u[m:m + 1])[0])
