"""Pins of the oracle's weight quantiser: block scale = mean absolute weight,
state = rint(clamp(w / scale, -1, 1)) (article "Neutrino-1: quantization is
a training decision, not a deployment one", "What's actually ternary").

The pins rest on values worked by hand, the exactly rounded mean of
math.fsum, and invariants of the definition (power-of-two scaling, sign
symmetry, one block per row)."""
import math

import numpy as np
import pytest

import oracle


def check_hand_worked(lib):
    # mean |w| = (0.5 + 1.5 + 0.25 + 2) / 4 = 1.0625; ratios 0.47, -1.41, 0.24, 1.88
    t, s = oracle.quantize_weights(np.array([[0.5, -1.5, 0.25, 2.0]], np.float32), 4, lib=lib)
    assert s.tolist() == [[1.0625]]
    assert t.tolist() == [[0, -1, 0, 1]]


def check_ties_round_to_even(lib):
    # mean 1: ratios +-0.5 round to 0 (half to even), 1.5 clamps to 1
    t, s = oracle.quantize_weights(np.array([[0.5, 1.5], [-0.5, -1.5]], np.float32), 2, lib=lib)
    assert s.tolist() == [[1.0], [1.0]]
    assert t.tolist() == [[0, 1], [0, -1]]


def check_short_last_block(lib):
    # K = 5, B = 2: blocks {0, 1}, {2, 3}, {4}; means 2, 2, 0.75
    t, s = oracle.quantize_weights(np.array([[1.0, 3.0, -2.0, 2.0, -0.75]], np.float32), 2, lib=lib)
    assert s.tolist() == [[2.0, 2.0, 0.75]]
    assert t.tolist() == [[0, 1, -1, 1, -1]]


def check_zero_block(lib):
    t, s = oracle.quantize_weights(np.array([[0, 0, 0, 0, 1, -1, 0, 0]], np.float32), 4, lib=lib)
    assert s.tolist() == [[0.0, 0.5]]
    assert t.tolist() == [[0, 0, 0, 0, 1, -1, 0, 0]]


def check_scale_is_the_exact_mean(lib):
    rng = np.random.default_rng(3)
    for B in (64, 128, 1000, 4096):
        W = (rng.standard_normal((6, 4096)) * rng.uniform(0.01, 10, (6, 1))).astype(np.float32)
        t, s = oracle.quantize_weights(W, B, lib=lib)
        nb = -(-4096 // B)
        assert s.shape == (6, nb)
        for i in range(6):
            for b in range(nb):
                blk = W[i, b * B:(b + 1) * B].astype(np.float64)
                exact = np.float32(math.fsum(np.abs(blk)) / len(blk))
                assert abs(float(s[i, b]) - float(exact)) <= float(np.spacing(exact)), (B, i, b)
        assert set(np.unique(t).tolist()) <= {-1, 0, 1}


def check_invariants(lib):
    rng = np.random.default_rng(4)
    W = rng.standard_normal((5, 777)).astype(np.float32)
    t, s = oracle.quantize_weights(W, 100, lib=lib)
    for k in (-4, 3):  # power-of-two scaling is exact all the way through
        t2, s2 = oracle.quantize_weights(W * np.float32(2.0 ** k), 100, lib=lib)
        assert np.array_equal(t2, t) and np.array_equal(s2, s * np.float32(2.0 ** k))
    tn, sn = oracle.quantize_weights(-W, 100, lib=lib)
    assert np.array_equal(tn, -t) and np.array_equal(sn, s)
    # B >= K: one scale per row, the row's mean absolute value
    t1, s1 = oracle.quantize_weights(W, 1000, lib=lib)
    assert s1.shape == (5, 1)
    for i in range(5):
        assert abs(float(s1[i, 0]) - math.fsum(np.abs(W[i].astype(np.float64))) / 777) <= 1e-6 * float(s1[i, 0])
    # about a third of standard-normal weights fall in (-scale / 2, scale / 2)
    assert 0.2 < float(np.mean(t == 0)) < 0.45
    # the states pack without a bad value
    assert oracle.pack(t, lib=lib)[2] == 0


WQUANT_CHECKS = [check_hand_worked, check_ties_round_to_even, check_short_last_block, check_zero_block,
                 check_scale_is_the_exact_mean, check_invariants]


@pytest.mark.parametrize("check", WQUANT_CHECKS, ids=lambda c: c.__name__)
def test_weight_quantiser_pin(check):
    check(oracle.load())
