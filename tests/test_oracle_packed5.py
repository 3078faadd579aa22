"""Pins of the oracle's 1.6-bit layout (five weights per byte) and of the
linear layer on it.

Each check rests on something other than the oracle's own formulas: rows
worked by hand (tests/golden/packed5_rows.txt), a second decoder derived
independently (digits read off by repeated tripling of the byte as a fraction
of 256), brute force over every pattern of five weights, and the already
pinned 2-bit layer on the same matrices."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "packed5_rows.txt")


def _weights(field):
    out = []
    for tok in field.split(","):
        if "*" in tok:
            n, x = tok.split("*")
            out += [int(x)] * int(n)
        else:
            out.append(int(tok))
    return out


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            K, w, hexrow, rs = line.split("|")
            rows.append((int(K), _weights(w), bytes.fromhex(hexrow), int(rs)))
    return rows


def _digits_by_tripling(b):
    # b / 256 read as a fraction: tripling it pushes the next base-3 digit
    # above the binary point (digit 0, the most significant, comes first)
    x, out = int(b), []
    for _ in range(5):
        x *= 3
        out.append(x >> 8)
        x &= 255
    return out


def _ternary(rng, N, K, p0=0.626):
    p = (1 - p0) / 2
    return rng.choice(np.array([-1, 0, 1], np.int8), p=[p, p0, p], size=(N, K))


# ---------------------------------------------------------------- checks --
# Each takes the oracle library so the mutation tests can run them on a
# deliberately broken copy.

def check_golden_rows5(lib):
    rows = _golden()
    assert len(rows) >= 8
    for K, w, row, rs in rows:
        assert len(w) == K
        assert oracle.row_bytes5(K, lib) == len(row)
        packed, rowsum, bad = oracle.pack5(np.array([w], np.int8), lib=lib)
        assert bad == 0
        assert packed.tobytes() == row, (K, packed.tobytes().hex(), row.hex())
        assert rowsum[0] == rs
        assert oracle.unpack5(np.frombuffer(row, np.uint8), 1, K, lib=lib)[0].tolist() == w


def check_every_byte_decodes(lib):
    # all 256 byte values, each at each of the four positions of a word:
    # digits from the tripling decoder, weight = digit - 1
    for n in range(4):
        packed = np.full((256, 16), 0x80, np.uint8)
        packed[:, n] = np.arange(256)
        w = oracle.unpack5(packed, 256, 20, lib=lib)
        for b in range(256):
            d = _digits_by_tripling(b)
            assert all(0 <= x <= 2 for x in d)
            assert [int(w[b, 4 * i + n]) for i in range(5)] == [x - 1 for x in d], (n, b)
            # the other bytes of the word are padding: weight 0
            others = [j for j in range(20) if j % 4 != n]
            assert not w[b, others].any()


def check_every_pattern_roundtrips(lib):
    # brute force: all 3^5 patterns of five weights at each byte position
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T
    assert pats.shape == (243, 5)
    for n in range(4):
        w = np.zeros((243, 20), np.int8)
        for i in range(5):
            w[:, 4 * i + n] = pats[:, i]
        packed, rowsum, bad = oracle.pack5(w, lib=lib)
        assert bad == 0
        assert np.array_equal(rowsum, pats.sum(1))
        assert np.array_equal(oracle.unpack5(packed, 243, 20, lib=lib), w)
        # one byte per pattern, all distinct; the rest of the row is padding
        assert len(set(packed[:, n].tolist())) == 243
        rest = np.delete(packed, n, axis=1)
        assert (rest == 0x80).all()
        # digits recovered by the tripling decoder
        for r in range(0, 243, 7):
            assert _digits_by_tripling(packed[r, n]) == [int(x) + 1 for x in pats[r]]
    # exactly 13 byte values are never written
    written = set()
    for n in range(1):
        w = np.zeros((243, 20), np.int8)
        for i in range(5):
            w[:, 4 * i] = pats[:, i]
        written |= set(oracle.pack5(w, lib=lib)[0][:, 0].tolist())
    assert len(set(range(256)) - written) == 13


def check_padding_is_weight_zero(lib):
    rng = np.random.default_rng(3)
    for K in (1, 19, 21, 79, 99, 161):
        w = _ternary(rng, 5, K)
        full = np.zeros((5, 80 * (-(-K // 80))), np.int8)
        full[:, :K] = w
        a, ra, _ = oracle.pack5(w, lib=lib)
        b, rb, _ = oracle.pack5(full, lib=lib)
        assert a.shape == b.shape
        assert np.array_equal(a, b) and np.array_equal(ra, rb)


def check_bad_values_counted(lib):
    w = np.array([[1, 2, -1, -5, 0, 1, 127, -128] + [0] * 20], np.int8)
    packed, rowsum, bad = oracle.pack5(w, lib=lib)
    assert bad == 4
    assert rowsum[0] == 1 - 1 + 1
    clean = np.where(np.abs(w) <= 1, w, 0).astype(np.int8)
    assert np.array_equal(packed, oracle.pack5(clean, lib=lib)[0])


def check_linear5_is_the_2bit_layer(lib):
    # the same matrix in both layouts gives the same int32 and fp32 results
    rng = np.random.default_rng(11)
    for K, M in ((1, 1), (19, 2), (20, 1), (21, 3), (80, 1), (81, 2), (100, 4), (1000, 2),
                 (4096, 1)):
        N = 33
        w = _ternary(rng, N, K)
        p5, rs5, _ = oracle.pack5(w, lib=lib)
        p2, rs2, _ = oracle.pack(w, lib=lib)
        assert np.array_equal(rs5, rs2)
        q = rng.integers(-128, 128, (M, K)).astype(np.int8)
        q[0, 0] = -128
        s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
        s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
        z = rng.integers(-8, 9, M).astype(np.int32)
        z[0] = 3
        a5, y5, d5 = oracle.linear5(p5, s_row, rs5, K, q, s_act, z, lib=lib)
        a2, y2, d2 = oracle.linear(p2, s_row, rs2, K, q, s_act, z, lib=lib)
        assert np.array_equal(a5, a2), K
        assert np.array_equal(y5.view(np.uint32), y2.view(np.uint32)), K
        assert np.array_equal(d5, d2), K


def check_linear5_against_integer_matmul(lib):
    rng = np.random.default_rng(5)
    N, K, M = 40, 333, 3
    w = _ternary(rng, N, K)
    p5, rs, _ = oracle.pack5(w, lib=lib)
    q = rng.integers(-128, 128, (M, K)).astype(np.int8)
    z = np.array([3, -7, 0], np.int32)
    acc, _, _ = oracle.linear5(p5, np.ones(N, np.float32), rs, K, q, 1.0, z, lib=lib)
    ref = (q.astype(np.int64) - z[:, None]) @ w.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)


def check_linear5_overflow_reported(lib):
    K = 140000  # 127 * K passes 2^24
    packed, rs, _ = oracle.pack5(np.ones((1, K), np.int8), lib=lib)
    with pytest.raises(ValueError):
        oracle.linear5(packed, [1.0], rs, K, np.full((1, K), 127, np.int8), 1.0, 0, lib=lib)
    K = 132104  # 127 * K = 2^24 - 8: still exact
    packed, rs, _ = oracle.pack5(np.ones((1, K), np.int8), lib=lib)
    acc, _, _ = oracle.linear5(packed, [1.0], rs, K, np.full((1, K), 127, np.int8), 1.0, 0,
                               lib=lib)
    assert acc[0, 0] == 127 * K


PACK5_CHECKS = [check_golden_rows5, check_every_byte_decodes, check_every_pattern_roundtrips,
                check_padding_is_weight_zero, check_bad_values_counted,
                check_linear5_is_the_2bit_layer, check_linear5_against_integer_matmul,
                check_linear5_overflow_reported]


@pytest.mark.parametrize("check", PACK5_CHECKS, ids=lambda c: c.__name__)
def test_packed5_pin(check):
    check(oracle.load())
