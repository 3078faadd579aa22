"""Pins of the oracle's neighbours of the ternary linear: the int8 output
head, the per-token activation quantiser and block-wise scales along K.

Each check rests on something other than the oracle's own formula: values
worked by hand, closed forms and invariants, a reduction to numpy's integer
matmul, the already-pinned per-row oracle, and the error bound of fp32
summation."""
import numpy as np
import pytest

import oracle

U = 2.0 ** -24  # fp32 unit roundoff


# ------------------------------------------------------------ quantiser --

def test_quantize_hand_worked():
    # lo = -1, hi = 2: s = 3/255; z = -128 - rint(-85) = -43;
    # q = rint(x / s) + z: -85-43 = -128, 0-43 = -43, rint(42.5) = 42 (half to
    # even) -> -1, 170-43 = 127
    q, s, z = oracle.quantize_act(np.array([[-1.0, 0.0, 0.5, 2.0]], np.float32))
    assert s[0] == np.float32(3.0) / np.float32(255.0)
    assert z[0] == -43
    assert q.tolist() == [[-128, -43, -1, 127]]


def test_quantize_special_tokens():
    x = np.zeros((4, 37), np.float32)
    x[1] = 3.5          # constant positive: range [0, 3.5]
    x[2] = -2.0         # constant negative: range [-2, 0]
    x[3, 5] = 1e-30     # one tiny value
    q, s, z = oracle.quantize_act(x)
    # all zeros: s = 1, z = -128, every code -128 (and s * (q - z) = 0)
    assert s[0] == 1.0 and z[0] == -128 and (q[0] == -128).all()
    # constant c > 0: lo = 0 -> z = -128, every x = hi -> code 127
    assert z[1] == -128 and (q[1] == 127).all()
    assert s[1] == np.float32(3.5) / np.float32(255.0)
    # constant c < 0: hi = 0 -> z = 127 - ... lo/s = -255 -> z = 127, x = lo -> -128
    assert z[2] == 127 and (q[2] == -128).all()
    # zeros of a token map exactly to its zero point
    assert (q[3][np.arange(37) != 5] == z[3]).all()


@pytest.mark.parametrize("seed", range(6))
def test_quantize_invariants(seed):
    rng = np.random.default_rng(seed)
    M, K = 5, 1000 + 37 * seed
    kind = seed % 3
    if kind == 0:
        x = rng.normal(0, 3, (M, K))
    elif kind == 1:
        x = rng.uniform(0.5, 9.0, (M, K))     # all positive
    else:
        x = -rng.exponential(2.0, (M, K))     # all negative
    x = x.astype(np.float32)
    x[:, 7] = 0.0
    q, s, z = oracle.quantize_act(x)
    assert (np.abs(z) <= 128).all()
    for m in range(M):
        xm = x[m].astype(np.float64)
        lo, hi = min(0.0, xm.min()), max(0.0, xm.max())
        # the scale spans the widened range in 255 steps
        assert abs(float(s[m]) * 255.0 - (hi - lo)) <= 1e-6 * (hi - lo)
        rec = float(s[m]) * (q[m].astype(np.float64) - z[m])
        # every value is reconstructed to within half a step (plus the fp32
        # rounding of x / s)
        assert np.all(np.abs(rec - xm) <= 0.5 * float(s[m]) * (1 + 1e-5) + 1e-6 * np.abs(xm))
        # zero is exact, the smallest value takes the lowest code when it is
        # below zero
        assert q[m, 7] == z[m]
        if xm.min() < 0:
            assert q[m, int(np.argmin(xm))] == -128
        # codes are monotone in x
        o = np.argsort(xm, kind="stable")
        assert np.all(np.diff(q[m][o].astype(np.int32)) >= 0)


def test_quantize_power_of_two_scaling():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (3, 513)).astype(np.float32)
    q0, s0, z0 = oracle.quantize_act(x)
    for k in (-3, 5):
        q1, s1, z1 = oracle.quantize_act(x * np.float32(2.0 ** k))
        assert np.array_equal(q0, q1) and np.array_equal(z0, z1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


# ----------------------------------------------------------- output head --

def test_head_hand_worked():
    W = np.array([[1, -2, 3], [127, -128, 0]], np.int8)
    rs = oracle.head_rowsum(W)
    assert rs.tolist() == [2, -1]
    acc, y32, y64 = oracle.head(W, [0.5, 0.25], rs, [[10, -20, 30]], 0.1, 3)
    # 10 + 40 + 90 - 3*2 = 134;  1270 + 2560 - 3*(-1) = 3833
    assert acc.tolist() == [[134, 3833]]
    assert abs(y64[0, 0] - 0.5 * 134 * np.float64(np.float32(0.1))) < 1e-12


@pytest.mark.parametrize("M,K", [(1, 64), (3, 1000), (8, 4096)])
def test_head_against_integer_matmul(M, K):
    rng = np.random.default_rng(M * 7 + K)
    N = 50
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    z = rng.integers(-128, 129, M).astype(np.int32)
    s_row = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    s_act = rng.uniform(0.01, 0.05, M).astype(np.float32)
    rs = oracle.head_rowsum(W)
    assert np.array_equal(rs, W.astype(np.int64).sum(1))
    acc, y32, y64 = oracle.head(W, s_row, rs, q, s_act, z)
    # sum_j W_ij (q_mj - z_m): numpy's int64 matmul, no row sums involved
    ref = (q.astype(np.int64) - z[:, None]) @ W.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)
    exact = s_row[None, :].astype(np.float64) * ref * s_act[:, None].astype(np.float64)
    assert np.allclose(y64, exact, rtol=1e-15, atol=0)
    # three fp32 roundings: int -> float, two products
    assert np.all(np.abs(y32.astype(np.float64) - exact) <= 3.01 * U * np.abs(exact))


def test_head_int_to_float_rounding():
    # acc = 1040 * 127 * 127 + 127 * 24 + 1 * 9 = 16,777,217 = 2^24 + 1, which
    # float rounds (to even) to 2^24; with s_row = 3 the three-rounding result
    # is 3 * 2^24 = 50,331,648, while rounding 3 * (2^24 + 1) once would give
    # 50,331,652 (fp32 spacing 4 there)
    W = np.array([[127] * 1040 + [127, 1]], np.int8)
    q = np.array([[127] * 1040 + [24, 9]], np.int8)
    acc, y32, _ = oracle.head(W, [3.0], oracle.head_rowsum(W), q, 1.0, 0)
    assert acc[0, 0] == 2 ** 24 + 1
    assert y32[0, 0] == np.float32(50331648.0)


def test_head_overflow_reported():
    # acc = K * (-128 * 127) - (-128) * (K * -128) = -32640 K, past -2^31
    K = 70000
    W = np.full((1, K), -128, np.int8)
    q = np.full((1, K), 127, np.int8)
    with pytest.raises(ValueError):
        oracle.head(W, [1.0], oracle.head_rowsum(W), q, 1.0, -128)
    # one column fewer than 2^31 / 32640 still fits
    K = 65792
    acc, _, _ = oracle.head(np.full((1, K), -128, np.int8), [1.0],
                            oracle.head_rowsum(np.full((1, K), -128, np.int8)),
                            np.full((1, K), 127, np.int8), 1.0, -128)
    assert acc[0, 0] == -32640 * K


# ----------------------------------------------------- block-wise scales --

def _ternary(rng, N, K, p0=0.6):
    p = (1 - p0) / 2
    return rng.choice(np.array([-1, 0, 1], np.int8), p=[p, p0, p], size=(N, K))


@pytest.mark.parametrize("K", [64, 100, 4096])
def test_one_block_is_the_per_row_layer(K):
    rng = np.random.default_rng(K)
    N, M = 40, 3
    w = _ternary(rng, N, K)
    packed, rowsum, bad = oracle.pack(w)
    assert bad == 0
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
    z = rng.integers(-8, 9, M).astype(np.int32)
    for B in (K, 4 * K):  # one block (B may exceed K)
        rb = oracle.block_rowsum(w, B)
        assert np.array_equal(rb[:, 0], rowsum)
        y32, y64, _ = oracle.linear_blocked(packed, s_row[:, None], rb, K, B, q, s_act, z)
        _, ry32, ry64 = oracle.linear(packed, s_row, rowsum, K, q, s_act, z)
        assert np.array_equal(y32.view(np.uint32), ry32.view(np.uint32))
        assert np.allclose(y64, ry64, rtol=1e-15, atol=0)


@pytest.mark.parametrize("K,B", [(256, 64), (1000, 128), (4096, 256), (12288, 512), (130, 64)])
def test_blocked_against_integer_sums(K, B):
    rng = np.random.default_rng(K + B)
    N, M = 30, 2
    w = _ternary(rng, N, K)
    packed, rowsum, _ = oracle.pack(w)
    nb = -(-K // B)
    rb = oracle.block_rowsum(w, B)
    assert rb.shape == (N, nb)
    assert np.array_equal(rb.sum(1), rowsum)
    for b in range(nb):
        assert np.array_equal(rb[:, b], w[:, b * B:(b + 1) * B].astype(np.int64).sum(1))
    s_b = rng.uniform(0.01, 0.1, (N, nb)).astype(np.float32)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
    z = rng.integers(-8, 9, M).astype(np.int32)
    y32, y64, yabs = oracle.linear_blocked(packed, s_b, rb, K, B, q, s_act, z)
    # per-block integer sums by numpy on the unpacked weights, q - z per token
    exact = np.zeros((M, N))
    mag = np.zeros((M, N))
    qz = q.astype(np.int64) - z[:, None]
    for b in range(nb):
        a = qz[:, b * B:(b + 1) * B] @ w[:, b * B:(b + 1) * B].astype(np.int64).T
        t = a * s_b[:, b].astype(np.float64)[None, :]
        exact += t
        mag += np.abs(t)
    exact *= s_act.astype(np.float64)[:, None]
    mag *= np.abs(s_act.astype(np.float64))[:, None]
    assert np.allclose(y64, exact, rtol=1e-12, atol=1e-12 * mag.max())
    assert np.allclose(yabs, mag, rtol=1e-12, atol=0)
    # the fp32 reference order is within the summation bound
    assert np.all(np.abs(y32.astype(np.float64) - exact) <= (nb + 1) * U * mag * 1.001)


def test_blocked_equal_scales_reduce_to_row_scale():
    rng = np.random.default_rng(5)
    N, K, B, M = 20, 2048, 128, 2
    w = _ternary(rng, N, K)
    packed, rowsum, _ = oracle.pack(w)
    rb = oracle.block_rowsum(w, B)
    s = rng.uniform(0.01, 0.1, N).astype(np.float32)
    s_b = np.repeat(s[:, None], K // B, axis=1)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    s_act = np.array([0.02, 0.03], np.float32)
    z = np.array([3, -5], np.int32)
    _, y64, _ = oracle.linear_blocked(packed, s_b, rb, K, B, q, s_act, z)
    _, _, ry64 = oracle.linear(packed, s, rowsum, K, q, s_act, z)
    assert np.allclose(y64, ry64, rtol=1e-13, atol=0)
