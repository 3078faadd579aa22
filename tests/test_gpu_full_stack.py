"""Full-size parity: the whole 8B-shaped stack (252 linears, 6.95 G weights,
1,400,832 output rows) in the launch configuration the benchmark times, at
M = 1 and M = 8, y only (the benchmark's configuration: at M = 8 the outputs
are held in registers until each workgroup's run ends) and with acc, and at
M = 16 (y only).  Every
output row of every linear is compared with the oracle, which recomputes
each linear from the same seeded weights and activations; every packed byte
and row sum is compared too.  The stack is also run with the input sharing
of a real layer (q/k/v and gate/up reading one activation buffer each)."""
import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import RTOL  # noqa: E402

SEED = 0
CHUNKS = 6  # layers are checked in six groups of six


@pytest.fixture(scope="module")
def runs():
    """Device stack, and host copies of y (and acc) of each configuration
    after two back-to-back launches of its plan."""
    from packed_bit_gemv_tern_amd.stack import DeviceStack
    st = DeviceStack("8b", seed=SEED, threads=16)
    out = {}
    for M, with_acc, share in [(1, True, False), (8, True, False), (1, False, False), (8, False, False),
                               (8, False, True), (16, False, False)]:
        b = st.bind(M, with_acc=with_acc, share_inputs=share)
        assert b.plan.L == 252
        assert b.plan.splits == 0  # a full stack keeps every linear whole
        b.run()
        b.run()
        torch.cuda.synchronize()
        out[(M, with_acc, share)] = ([y.cpu().numpy() for y in b.y],
                                     [a.cpu().numpy() for a in b.acc] if with_acc else None,
                                     b.plan.restages)
        del b
        torch.cuda.empty_cache()
    yield st, out
    del st
    torch.cuda.empty_cache()


def _check(y, ry32, ry64, ctx):
    assert np.all(np.abs(y.astype(np.float64) - ry64) <= RTOL * np.abs(ry64)), ctx
    assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), ctx


@pytest.mark.timeout(300)
@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_full_8b_stack_every_row(runs, chunk):
    st, out = runs
    specs = st.specs
    per = len(specs) // CHUNKS
    rows = 0
    for i in range(chunk * per, (chunk + 1) * per):
        layer, idx, name, N, K, p0 = specs[i]
        pl = st.linears[i]
        w, s_row = synth.make_weights(SEED, layer, idx, N, K, p0)
        rp, rr, bad = oracle.pack(w)
        assert bad == 0
        assert np.array_equal(pl.packed.cpu().numpy(), rp), pl.name
        assert np.array_equal(pl.rowsum.cpu().numpy(), rr), pl.name
        for M in (1, 8):
            q, s_act, z = synth.make_activations(SEED, layer, idx, K, M)
            racc, ry32, ry64 = oracle.linear(rp, s_row, rr, K, q, s_act, z)
            ys, accs, _ = out[(M, True, False)]
            assert np.array_equal(accs[i], racc), (pl.name, M)
            _check(ys[i], ry32, ry64, (pl.name, M, "with acc"))
            ys, _, _ = out[(M, False, False)]
            _check(ys[i], ry32, ry64, (pl.name, M, "y only"))
        # 16 tokens (the 16-token window kernel), y only
        q, s_act, z = synth.make_activations(SEED, layer, idx, K, 16)
        _, ry32, ry64 = oracle.linear(rp, s_row, rr, K, q, s_act, z)
        ys, _, _ = out[(16, False, False)]
        _check(ys[i], ry32, ry64, (pl.name, 16, "y only"))
        # q/k/v and gate/up sharing one input: the group's first linear's
        # activations
        src = synth.INPUT_LEADER[idx]
        q, s_act, z = synth.make_activations(SEED, layer, src, K, 8)
        _, ry32, ry64 = oracle.linear(rp, s_row, rr, K, q, s_act, z)
        ys, _, _ = out[(8, False, True)]
        _check(ys[i], ry32, ry64, (pl.name, 8, "shared inputs"))
        rows += N
    assert rows == sum(s[3] for s in specs[chunk * per:(chunk + 1) * per])


def test_full_8b_stack_shared_inputs_restage_less(runs):
    _, out = runs
    # 36 layers x (q/k/v + gate/up): sharing saves window loads
    assert out[(8, False, True)][2] < out[(8, False, False)][2]


@pytest.fixture(scope="module")
def layer8b():
    from packed_bit_gemv_tern_amd.stack import DeviceStack
    st = DeviceStack("8b", layers=1, seed=3, threads=16, sample_rows=96)
    yield st
    del st
    torch.cuda.empty_cache()


def _check_sampled(st, b, M):
    for i, pl in enumerate(st.linears):
        rows = pl.sample_rows
        q, s_act, z = b.host_act[i]
        rp, rr, bad = oracle.pack(pl.sample_w)
        racc, ry32, ry64 = oracle.linear(rp, pl.sample_s_row, rr, pl.K, q, s_act, z)
        acc = b.acc[i].cpu().numpy()[:, rows]
        y = b.y[i].cpu().numpy()[:, rows]
        assert np.array_equal(acc, racc), (pl.name, M)
        assert np.all(np.abs(y.astype(np.float64) - ry64) <= RTOL * np.abs(ry64)), (pl.name, M)
        assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), (pl.name, M)


# M = 16: the 16-token window kernel (11); prefill GEMM variants: 9 = 128 x
# 64 tiles, 14 = 256 x 128, 10 = 512 x 128
@pytest.mark.timeout(300)
@pytest.mark.parametrize("M,kernel", [(16, 16 + 11), (64, 16 + 9), (512, 16 + 14)])
def test_8b_layer_prefill_sampled(layer8b, M, kernel):
    """One 8B layer as one stack launch at prefill M (the configuration the
    prefill sweep times): sampled rows of every linear against the oracle."""
    b = layer8b.bind(M, with_acc=True)
    assert b.plan.kernel == kernel, (M, b.plan.kernel)
    b.run()
    b.run()
    torch.cuda.synchronize()
    _check_sampled(layer8b, b, M)


@pytest.fixture(scope="module")
def layers8b4():
    from packed_bit_gemv_tern_amd.stack import DeviceStack
    st = DeviceStack("8b", layers=4, seed=3, threads=16, sample_rows=48)
    yield st
    del st
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M", [512, 300])
def test_8b_four_layers_prefill_sampled(layers8b4, M):
    """Four 8B layers (28 linears) as one launch at M = 512 (the profiled
    prefill workload) and at a ragged M = 300: enough tiles for the 512-row
    GEMM tile; sampled rows of every linear against the oracle."""
    b = layers8b4.bind(M, with_acc=True)
    assert b.plan.kernel == 16 + 10 and b.plan.splits == 0, (M, b.plan.kernel, b.plan.splits)
    b.run()
    b.run()
    torch.cuda.synchronize()
    _check_sampled(layers8b4, b, M)
