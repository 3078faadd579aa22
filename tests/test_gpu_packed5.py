"""The 1.6-bit layout (five weights per byte) on the GPU against the oracle:
packed bytes, row sums and bad-value counts bit-exact; acc and the fp32
output of the M = 1 linear bit-exact (same two roundings), on ragged K and
N, both lane shapes of the kernel, every byte value, and the full-width
8B gate and down shapes."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import synth, tern  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402


def _pack5_gpu(w, ldw=None):
    N, K = w.shape
    ldw = ldw or K
    wp = np.full((N, ldw), 5, np.int8)  # columns past K hold junk
    wp[:, :K] = w
    packed = torch.full((max(N, 1), tern.tern_row_bytes5(K)), 0xA5, dtype=torch.uint8, device=DEV)
    rs = torch.full((max(N, 1),), -9, dtype=torch.int32, device=DEV)
    bad = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    tern.tern_pack5(to_dev(wp), N, K, ldw, packed, rs, bad)
    torch.cuda.synchronize()
    return packed, rs, int(bad.item())


def _gemv5(packed, s_row, rs, N, K, q, s_act, z):
    y = torch.full((N + 5,), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((N + 5,), -7, dtype=torch.int32, device=DEV)
    qd = np.zeros((K + 15) // 16 * 16, np.int8)
    qd[:K] = q.reshape(-1)
    tern.tern_gemv5(packed, to_dev(s_row), rs, N, K, to_dev(qd), to_dev(np.asarray(s_act, np.float32).reshape(1)),
                    to_dev(np.asarray(z, np.int32).reshape(1)), y, acc)
    torch.cuda.synchronize()
    y, acc = y.cpu().numpy(), acc.cpu().numpy()
    assert np.isnan(y[N:]).all() and (acc[N:] == -7).all()  # nothing past N written
    return y[:N], acc[:N]


@pytest.mark.parametrize("K", [1, 4, 5, 19, 20, 21, 79, 80, 81, 100, 1000, 4096, 12288])
@pytest.mark.parametrize("N", [1, 7, 300])
def test_pack5_parity(N, K):
    rng = np.random.default_rng([N, K, 1])
    w = synth.ternary(rng, N, K, 0.626)
    w[rng.random((N, K)) < 0.01] = 3  # a few values outside {-1, 0, 1}
    packed, rs, bad = _pack5_gpu(w, ldw=K + 13)
    opk, ors, obad = oracle.pack5(w)
    assert np.array_equal(packed.cpu().numpy()[:N], opk)
    assert np.array_equal(rs.cpu().numpy()[:N], ors)
    assert bad == obad


# K = 4096 and 4100 take the 8-lane rows of the kernel, the others 16
@pytest.mark.parametrize("K", [1, 3, 19, 20, 21, 79, 80, 81, 100, 640, 1000, 1024, 1280, 2048, 3072,
                               4096, 4100, 12288, 16000])
@pytest.mark.parametrize("N", [1, 17, 300])
def test_gemv5_parity(N, K):
    rng = np.random.default_rng([N, K, 2])
    w = synth.ternary(rng, N, K, 0.626)
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    q = synth.activations(rng, 1, K)
    s_act, z = np.float32(0.02), np.int32(3)
    packed, rs, _ = _pack5_gpu(w)
    y, acc = _gemv5(packed, s_row, rs, N, K, q, s_act, z)
    opk, ors, _ = oracle.pack5(w)
    racc, ry32, ry64 = oracle.linear5(opk, s_row, ors, K, q, s_act, z)
    assert np.array_equal(acc, racc[0]), (N, K)
    assert np.array_equal(y.view(np.uint32), ry32[0].view(np.uint32)), (N, K)
    assert np.allclose(y, ry64[0], rtol=1e-6, atol=0)


@pytest.mark.parametrize("K", [20, 100, 4096])
def test_gemv5_every_byte_value(K):
    # arbitrary bytes, the 13 never-written values included, with the row
    # sums of what they decode to
    N = 256
    ld = tern.tern_row_bytes5(K)
    rng = np.random.default_rng([K, 3])
    raw = rng.integers(0, 256, (N, ld), dtype=np.uint8)
    raw[:, 0] = np.arange(256)
    w = oracle.unpack5(raw, N, K)
    rs = w.astype(np.int64).sum(1).astype(np.int32)
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    q = synth.activations(rng, 1, K)
    y, acc = _gemv5(to_dev(raw), s_row, to_dev(rs), N, K, q, np.float32(0.015), np.int32(-5))
    racc, ry32, _ = oracle.linear5(raw, s_row, rs, K, q, np.float32(0.015), np.int32(-5))
    assert np.array_equal(acc, racc[0])
    assert np.array_equal(y.view(np.uint32), ry32[0].view(np.uint32))


@pytest.mark.parametrize("case", ["plus_max", "minus_min", "zero_point_max", "mixed"])
def test_gemv5_extremes(case):
    N, K = 33, 3000
    rng = np.random.default_rng(7)
    if case == "plus_max":
        w, q, z = np.ones((N, K), np.int8), np.full((1, K), 127, np.int8), 0
    elif case == "minus_min":
        w, q, z = -np.ones((N, K), np.int8), np.full((1, K), -128, np.int8), 0
    elif case == "zero_point_max":
        w, q, z = synth.ternary(rng, N, K, 0.2), synth.activations(rng, 1, K), 255
    else:
        w, q, z = synth.ternary(rng, N, K, 0.0), synth.activations(rng, 1, K), -255
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    packed, rs, _ = _pack5_gpu(w)
    y, acc = _gemv5(packed, s_row, rs, N, K, q, np.float32(0.02), np.int32(z))
    opk, ors, _ = oracle.pack5(w)
    racc, ry32, _ = oracle.linear5(opk, s_row, ors, K, q, np.float32(0.02), np.int32(z))
    assert np.array_equal(acc, racc[0])
    assert np.array_equal(y.view(np.uint32), ry32[0].view(np.uint32))


def test_gemv5_widest_K():
    N, K = 9, tern.TERN5_MAX_K
    rng = np.random.default_rng(8)
    w = synth.ternary(rng, N, K, 0.626)
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    q = synth.activations(rng, 1, K)
    packed, rs, _ = _pack5_gpu(w)
    y, acc = _gemv5(packed, s_row, rs, N, K, q, np.float32(0.02), np.int32(3))
    opk, ors, _ = oracle.pack5(w)
    racc, ry32, _ = oracle.linear5(opk, s_row, ors, K, q, np.float32(0.02), np.int32(3))
    assert np.array_equal(acc, racc[0])
    assert np.array_equal(y.view(np.uint32), ry32[0].view(np.uint32))


@pytest.mark.parametrize("idx", [4, 6])  # the 8B gate (12,288 x 4,096) and down (4,096 x 12,288)
def test_gemv5_full_8b_linear_sampled(idx):
    layer = 2
    spec = [s for s in synth.stack_specs("8b") if s[0] == layer and s[1] == idx][0]
    _, _, name, N, K, p0 = spec
    w, s_row = synth.make_weights(0, layer, idx, N, K, p0)
    q, s_act, z = synth.make_activations(0, layer, idx, K, 1)
    packed, rs, bad = _pack5_gpu(w)
    assert bad == 0
    y, acc = _gemv5(packed, s_row, rs, N, K, q, s_act[0], z[0])
    rows = np.unique(np.concatenate([np.arange(0, N, 37), [N - 1]]))
    opk, ors, _ = oracle.pack5(w[rows])
    assert np.array_equal(packed.cpu().numpy()[rows], opk)
    racc, ry32, _ = oracle.linear5(opk, s_row[rows], ors, K, q, s_act, z)
    assert np.array_equal(acc[rows], racc[0])
    assert np.array_equal(y[rows].view(np.uint32), ry32[0].view(np.uint32))
