"""Pins of the CPU oracle against facts fixed by the pages, the layout's own
definition and the mathematics -- never against the oracle itself.

Each check is a function of the loaded oracle library so that
``test_oracle_mutants.py`` can run the same checks on deliberately broken
copies of the oracle and show that some pin catches every plausible slip.
"""
import itertools
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32_from_bits(h: str) -> np.float32:
    return np.frombuffer(struct.pack("<I", int(h, 16)), np.float32)[0]


def bits_of(x) -> str:
    return "%08x" % struct.unpack("<I", np.float32(x).tobytes())[0]


def read_packed_rows():
    cases = []
    with open(os.path.join(GOLDEN, "packed_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            K, ws, hx, rs = line.split("|")
            if "*" in ws:
                v, n = ws.split("*")
                w = [int(v)] * int(n)
            else:
                w = [int(v) for v in ws.split(",")]
            assert len(w) == int(K), line
            cases.append((int(K), np.array(w, np.int8), hx, int(rs)))
    return cases


def read_linear_case():
    d = {}
    with open(os.path.join(GOLDEN, "linear_case.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=", 1)
                d[k] = v
    return d


# ---------------------------------------------------------------- checks ---

def check_golden_rows(lib):
    for K, w, hx, rs in read_packed_rows():
        packed, rowsum, bad = oracle.pack(w[None, :], lib=lib)
        assert bad == 0
        assert packed.tobytes().hex() == hx, (K, w)
        assert int(rowsum[0]) == rs
        back, invalid = oracle.unpack(packed, 1, K, lib=lib)
        assert invalid == 0 and np.array_equal(back[0], w)
        assert oracle.validate(packed, 1, K, lib=lib) == (0, 0)


def check_golden_linear(lib):
    d = read_linear_case()
    K = int(d["K"])
    w = np.array([int(v) for v in d["w"].split(",")], np.int8)[None, :]
    q = np.array([int(v) for v in d["q"].split(",")], np.int8)[None, :]
    s_row = np.array([f32_from_bits(d["s_row_bits"])], np.float32)
    s_act = np.array([f32_from_bits(d["s_act_bits"])], np.float32)
    z = np.array([int(d["z"])], np.int32)
    packed, rowsum, _ = oracle.pack(w, lib=lib)
    assert int(rowsum[0]) == int(d["rowsum"])
    acc, y32, y64 = oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
    assert int(acc[0, 0]) == int(d["acc"])
    assert bits_of(y32[0, 0]) == d["y_bits"]
    # the hand-worked intermediate, by numpy's own IEEE float32 product
    assert bits_of(s_row[0] * np.float32(int(d["acc"]))) == d["t_bits"]
    assert y64[0, 0] == float(s_row[0]) * int(d["acc"]) * float(s_act[0])


def all_patterns(K):
    return np.array(list(itertools.product((-1, 0, 1), repeat=K)), np.int8)


def check_bruteforce(lib, kmax=8):
    """Every ternary row of width K <= kmax, against direct integer sums."""
    rng = np.random.default_rng(1234)
    for K in range(1, kmax + 1):
        W = all_patterns(K)
        packed, rowsum, bad = oracle.pack(W, lib=lib)
        assert bad == 0
        # no byte holds a 11 field
        b = packed.astype(np.int64)
        for s in (0, 2, 4, 6):
            assert not np.any(((b >> s) & 3) == 3)
        back, invalid = oracle.unpack(packed, W.shape[0], K, lib=lib)
        assert invalid == 0 and np.array_equal(back, W)
        assert np.array_equal(rowsum, W.astype(np.int64).sum(1))
        qs = [rng.integers(-128, 128, K), np.full(K, -128), np.full(K, 127),
              np.eye(K, dtype=np.int64)[K // 2] * 77]
        zs = [-128, 0, 3, 127]
        q = np.array([qv for qv in qs for _ in zs], np.int8)
        z = np.array([zv for _ in qs for zv in zs], np.int32)
        s_row = np.full(W.shape[0], 0.5, np.float32)
        s_act = np.full(q.shape[0], 0.25, np.float32)
        acc, _, _ = oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
        Wl = W.astype(np.int64)
        for m in range(q.shape[0]):
            direct = (Wl * q[m].astype(np.int64)).sum(1) - int(z[m]) * Wl.sum(1)
            assert np.array_equal(acc[m].astype(np.int64), direct), (K, m)


def check_roundtrip_random(lib):
    rng = np.random.default_rng(5)
    for K in list(range(1, 131)) + [512, 1024, 2048, 3072, 4096]:
        W = synth.ternary(rng, 7, K, 0.626)
        packed, rowsum, bad = oracle.pack(W, lib=lib)
        assert bad == 0 and packed.shape == (7, 16 * ((K + 63) // 64))
        back, invalid = oracle.unpack(packed, 7, K, lib=lib)
        assert invalid == 0 and np.array_equal(back, W)
        assert oracle.validate(packed, 7, K, lib=lib) == (0, 0)
        assert np.array_equal(rowsum, W.astype(np.int64).sum(1))


def check_matmul(lib):
    """acc equals numpy's integer matmul of the unpacked weights, minus z * rowsum."""
    rng = np.random.default_rng(7)
    for (N, K, M) in [(37, 300, 5), (64, 4096, 3), (5, 12288, 2), (129, 65, 16)]:
        W = synth.ternary(rng, N, K, 0.626)
        q = rng.integers(-128, 128, (M, K)).astype(np.int8)
        z = rng.integers(-200, 200, M).astype(np.int32)
        s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
        s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
        packed, rowsum, _ = oracle.pack(W, lib=lib)
        acc, y32, y64 = oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
        ref = np.matmul(q.astype(np.int64), W.astype(np.int64).T) \
            - z.astype(np.int64)[:, None] * W.astype(np.int64).sum(1)[None, :]
        assert np.array_equal(acc.astype(np.int64), ref)
        y_ref = s_row.astype(np.float64)[None, :] * ref * s_act.astype(np.float64)[:, None]
        np.testing.assert_allclose(y64, y_ref, rtol=1e-15, atol=0)


def check_two_formulas(lib):
    """sum_j w (q - z) (no packing, no stored row sum) equals the packed path."""
    rng = np.random.default_rng(11)
    for (N, K, M) in [(50, 777, 4), (8, 4096, 8)]:
        W = synth.ternary(rng, N, K, 0.626)
        q = rng.integers(-128, 128, (M, K)).astype(np.int8)
        z = rng.integers(-8, 9, M).astype(np.int32)
        s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
        s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
        packed, rowsum, _ = oracle.pack(W, lib=lib)
        acc, _, y64 = oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
        acc2, y64b = oracle.linear_direct(W, s_row, q, s_act, z, lib=lib)
        assert np.array_equal(acc.astype(np.int64), acc2)
        assert np.array_equal(y64, y64b)


def check_closed_forms(lib):
    rng = np.random.default_rng(13)
    K = 200
    q = rng.integers(-128, 128, (3, K)).astype(np.int8)
    z = np.array([-5, 0, 9], np.int32)
    s_act = np.array([0.02, 0.03, 0.01], np.float32)
    # W = 0: acc = 0 and y = +0.0 exactly
    W = np.zeros((9, K), np.int8)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    acc, y32, y64 = oracle.linear(packed, np.full(9, 0.07, np.float32), rowsum, K, q, s_act, z, lib=lib)
    assert not acc.any() and not y32.any() and not np.signbit(y32).any()
    # q = c everywhere: acc = (c - z) * rowsum
    W = synth.ternary(rng, 40, K, 0.5)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    for c in (-128, -1, 0, 5, 127):
        qc = np.full((3, K), c, np.int8)
        acc, _, _ = oracle.linear(packed, np.ones(40, np.float32), rowsum, K, qc, s_act, z, lib=lib)
        assert np.array_equal(acc.astype(np.int64),
                              (c - z.astype(np.int64))[:, None] * W.astype(np.int64).sum(1)[None, :])
    # W = +I: acc_i = q_i - z;  W = -I: acc_i = z - q_i
    for sign in (1, -1):
        W = (sign * np.eye(K)).astype(np.int8)
        packed, rowsum, _ = oracle.pack(W, lib=lib)
        acc, _, _ = oracle.linear(packed, np.ones(K, np.float32), rowsum, K, q, s_act, z, lib=lib)
        assert np.array_equal(acc.astype(np.int64),
                              sign * (q.astype(np.int64) - z.astype(np.int64)[:, None]))
    # z = 0 and a one-hot q select a column: acc = W[:, j] * q_j
    W = synth.ternary(rng, 33, K, 0.626)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    for j in (0, 63, 64, 150, K - 1):
        qj = np.zeros((1, K), np.int8)
        qj[0, j] = -77
        acc, _, _ = oracle.linear(packed, np.ones(33, np.float32), rowsum, K, qj, [1.0], [0], lib=lib)
        assert np.array_equal(acc[0], W[:, j].astype(np.int32) * -77)


def check_fp32_epilogue(lib):
    """y32 = (s_row * acc) * s_act with two IEEE float32 roundings, checked
    against numpy's float32 products and against exact rationals."""
    rng = np.random.default_rng(17)
    N, K, M = 300, 4096, 4
    W = synth.ternary(rng, N, K, 0.626)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    z = rng.integers(-8, 9, M).astype(np.int32)
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    acc, y32, y64 = oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
    t = s_row[None, :] * acc.astype(np.float32)
    y_np = t * s_act[:, None]
    assert y_np.dtype == np.float32
    assert np.array_equal(y32.view(np.uint32), y_np.view(np.uint32))
    for (m, i) in [(0, 0), (1, 17), (3, 299), (2, 150)]:
        exact = Fraction(float(s_row[i])) * int(acc[m, i]) * Fraction(float(s_act[m]))
        if exact == 0:
            continue
        assert abs(Fraction(float(y64[m, i])) - exact) <= abs(exact) * Fraction(1, 2 ** 52)
        assert abs(Fraction(float(y32[m, i])) - exact) <= abs(exact) * Fraction(1, 2 ** 23)


def check_invalid_codes(lib):
    W = np.array([[1, 0, -1, 0, 1]], np.int8)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    bad = packed.copy()
    bad[0, 2] |= 0x03          # weight 2 (byte 2, bit 0) -> 11
    _, invalid = oracle.unpack(bad, 1, 5, lib=lib)
    assert invalid == 1
    assert oracle.validate(bad, 1, 5, lib=lib) == (1, 0)
    with pytest.raises(ValueError):
        oracle.linear(bad, [1.0], rowsum, 5, np.zeros((1, 5), np.int8), [1.0], [0], lib=lib)
    pad = packed.copy()
    pad[0, 5] = 0x54           # weight 5 is padding; 00 instead of 01
    assert oracle.validate(pad, 1, 5, lib=lib) == (0, 1)
    _, invalid = oracle.unpack(pad, 1, 5, lib=lib)
    assert invalid == 0


def check_bad_pack_values(lib):
    W = np.array([[1, 2, 0, -5, -1, 127]], np.int8)
    _, rowsum, bad = oracle.pack(W, lib=lib)
    assert bad == 3 and int(rowsum[0]) == 0


def check_overflow(lib):
    K = 1 << 17
    W = np.ones((1, K), np.int8)
    packed, rowsum, _ = oracle.pack(W, lib=lib)
    q = np.full((1, K), -128, np.int8)
    with pytest.raises(ValueError):
        oracle.linear(packed, [1.0], rowsum, K, q, [1.0], [127], lib=lib)
    acc, _, _ = oracle.linear(packed, [1.0], rowsum, K, q, [1.0], [127], lib=lib, check=False)
    # the int32 store of an out-of-range acc is not trusted; only the status is


ALL_CHECKS = [check_golden_rows, check_golden_linear, check_bruteforce, check_roundtrip_random,
              check_matmul, check_two_formulas, check_closed_forms, check_fp32_epilogue,
              check_invalid_codes, check_bad_pack_values, check_overflow]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)


def test_row_bytes():
    # four weights per byte, rows rounded up to 16-byte chunks of 64 weights
    for K, ld in [(1, 16), (63, 16), (64, 16), (65, 32), (512, 128), (1024, 256),
                  (2048, 512), (3072, 768), (4096, 1024), (12288, 3072)]:
        assert oracle.row_bytes(K) == ld
