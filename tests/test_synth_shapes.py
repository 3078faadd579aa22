"""The synthetic workloads' shapes and state mix against figures the pages print."""
import numpy as np

from packed_bit_gemv_tern_amd import synth


def _weights(model):
    return sum(N * K for (_, _, _, N, K, _) in synth.stack_specs(model))


def test_8b_shapes_match_parameter_count():
    # Neutrino-1 8B model card, "Architecture": 8,190,735,360 parameters, of
    # which two untied int8 tables of 151,936 x 4,096 and fp32 norms: 4 per
    # layer (two RMSNorms of 4,096, per-head q/k norms of 128) plus the final
    # norm -- 145 tensors.
    norms = 36 * (4096 + 4096 + 128 + 128) + 4096
    assert 36 * 4 + 1 == 145
    assert _weights("8b") == 8_190_735_360 - 2 * 151_936 * 4096 - norms
    assert _weights("8b") == 6_945_767_424          # "6.95B coded projection weights"
    assert len(synth.stack_specs("8b")) == 252      # "252 transformer linears"
    assert sum(N for (_, _, _, N, _, _) in synth.stack_specs("8b")) == 1_400_832


def test_06b_shapes_match_parameter_count():
    # Fermion Research models page, "Neutrino-1 0.6B": 596,049,920 parameters,
    # one tied int8 table of 151,936 x 1,024, 196 transformer linears, coded
    # lane 73.9 % of the parameters.
    norms = 28 * (1024 + 1024 + 128 + 128) + 1024
    total = 596_049_920
    assert _weights("0.6b") == total - 151_936 * 1024 - norms == 440_401_920
    assert len(synth.stack_specs("0.6b")) == 196
    assert round(100 * _weights("0.6b") / total, 1) == 73.9


def test_single_gemv_case_distribution():
    lin = synth.single_gemv_case()
    assert lin.w.shape == (256, 512) and lin.q.shape == (1, 512)
    assert set(np.unique(lin.w)) <= {-1, 0, 1}
    zero = (lin.w == 0).mean()
    assert abs(zero - 0.626) < 0.01
    assert 0.01 <= lin.s_row.min() and lin.s_row.max() < 0.1
    assert lin.s_act[0] == np.float32(0.02) and lin.z[0] == 3


def test_stack_linear_distribution_and_determinism():
    a = synth.make_linear(0, 2, 6, 4096, 12288, synth.zero_rate_8b(2, "down"), 8)
    b = synth.make_linear(0, 2, 6, 4096, 12288, synth.zero_rate_8b(2, "down"), 8)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.q, b.q)
    zero = (a.w == 0).mean()
    assert abs(zero - 0.7247) < 0.002
    plus, minus = (a.w == 1).mean(), (a.w == -1).mean()
    assert abs(plus - minus) < 0.002
    assert a.q.min() == -128 and a.q.max() == 127
    assert a.s_act.shape == (8,) and (-8 <= a.z).all() and (a.z <= 8).all()


def test_zero_rates_follow_pages():
    # attention flat near 62 %; gate / down spike in 0-based layers 1-3;
    # layer 0 down is the densest tensor at 60.59 % (article, "Sparsity is
    # learned, not imposed")
    assert synth.zero_rate_8b(17, "k") == 0.62
    assert synth.zero_rate_8b(2, "down") == 0.7247
    assert synth.zero_rate_8b(3, "gate") == 0.7048
    assert synth.zero_rate_8b(0, "down") == 0.6059
    rates = [p for (_, _, _, _, _, p) in synth.stack_specs("8b")]
    assert min(rates) == 0.6059


def test_make_stack_streams_in_order():
    seen = []
    synth.make_stack(0, 1, model="0.6b", layers=2, threads=3,
                     consume=lambda pos, lin: seen.append((pos, lin.w.shape)))
    assert [p for p, _ in seen] == list(range(14))
    assert seen[6][1] == (1024, 3072)
