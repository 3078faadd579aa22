"""Block-scaled ternary GEMV on the GPU against the oracle.  Block row sums are
integers (bit-exact).  y sums the scaled blocks in block order from +0 with
one rounding per product and per sum, as the oracle's fp32 evaluation does,
so it must equal that value bit for bit; it is also within the bound of fp32
summation, (nb + 1) * 2^-24 * |s_act| * sum_b |s_b acc_b|, of the exact
value."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import tern  # noqa: E402
from gpu_util import DEV, gpu_pack, to_dev  # noqa: E402

U = 2.0 ** -24


def _case(N, K, B, seed):
    rng = np.random.default_rng([seed, N, K, B])
    p = 0.187
    w = rng.choice(np.array([-1, 0, 1], np.int8), p=[p, 1 - 2 * p, p], size=(N, K))
    nb = -(-K // B)
    s_b = rng.uniform(0.01, 0.1, (N, nb)).astype(np.float32)
    q = rng.integers(-128, 128, (1, K), dtype=np.int8)
    s_act = np.array([rng.uniform(0.01, 0.03)], np.float32)
    z = np.array([rng.integers(-8, 9)], np.int32)
    return w, s_b, q, s_act, z, nb


def _run(w, s_b, q, s_act, z, B):
    N, K = w.shape
    packed, _, _ = gpu_pack(w)
    nb = s_b.shape[1]
    rb = torch.empty((N, nb), dtype=torch.int32, device=DEV)
    tern.tern_block_rowsum(packed, N, K, B, rb)
    qp = np.zeros((1, (K + 15) // 16 * 16), np.int8)
    qp[:, :K] = q
    y = torch.full((N + 4,), float("nan"), dtype=torch.float32, device=DEV)
    tern.tern_gemv_blocked(packed, to_dev(s_b), rb, N, K, B, to_dev(qp), to_dev(s_act), to_dev(z), y)
    torch.cuda.synchronize()
    return rb.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("B", [64, 128, 256, 1024, 4096])
@pytest.mark.parametrize("K", [64, 100, 576, 1024, 4096, 4160, 12288, 16384])
def test_blocked_parity(K, B):
    N = 37 if K >= 12288 else 300
    w, s_b, q, s_act, z, nb = _case(N, K, B, seed=1)
    rb, y = _run(w, s_b, q, s_act, z, B)
    assert np.array_equal(rb, oracle.block_rowsum(w, B))
    rp, _, _ = oracle.pack(w)
    y32, y64, yabs = oracle.linear_blocked(rp, s_b, oracle.block_rowsum(w, B), K, B, q, s_act, z)
    yg = y[:N].astype(np.float64)
    bound = (nb + 1) * U * yabs[0] * 1.001
    assert np.all(np.abs(yg - y64[0]) <= bound), (K, B)
    assert np.array_equal(y[:N].view(np.uint32), y32[0].view(np.uint32)), (K, B)
    assert np.isnan(y[N:]).all()  # nothing written past N


@pytest.mark.parametrize("N", [1, 2, 3, 5, 63, 1001])
def test_blocked_ragged_rows(N):
    K, B = 4096, 128
    w, s_b, q, s_act, z, nb = _case(N, K, B, seed=2)
    rb, y = _run(w, s_b, q, s_act, z, B)
    rp, _, _ = oracle.pack(w)
    y32, y64, yabs = oracle.linear_blocked(rp, s_b, rb, K, B, q, s_act, z)
    assert np.all(np.abs(y[:N].astype(np.float64) - y64[0]) <= (nb + 1) * U * yabs[0] * 1.001)
    assert np.array_equal(y[:N].view(np.uint32), y32[0].view(np.uint32))


def test_blocked_equal_scales_match_row_path():
    """Equal block scales: the per-row GEMV's result, within the bound."""
    N, K, B = 500, 12288, 256
    w, _, q, s_act, z, nb = _case(N, K, B, seed=3)
    s = np.random.default_rng(9).uniform(0.01, 0.1, N).astype(np.float32)
    s_b = np.repeat(s[:, None], nb, axis=1)
    rb, y = _run(w, s_b, q, s_act, z, B)
    rp, rr, _ = oracle.pack(w)
    _, _, ry64 = oracle.linear(rp, s, rr, K, q, s_act, z)
    _, _, yabs = oracle.linear_blocked(rp, s_b, rb, K, B, q, s_act, z)
    assert np.all(np.abs(y[:N].astype(np.float64) - ry64[0]) <= (nb + 1) * U * yabs[0] * 1.001)


def test_blocked_errors():
    lib = tern.library()
    p = torch.zeros((4, 64), dtype=torch.uint8, device=DEV)
    f = torch.zeros(64, dtype=torch.float32, device=DEV)
    i = torch.zeros(64, dtype=torch.int32, device=DEV)
    q = torch.zeros(64, dtype=torch.int8, device=DEV)

    def call(K, B):
        return lib.tern_gemv_blocked(p.data_ptr(), f.data_ptr(), i.data_ptr(), 4, K, B, q.data_ptr(),
                                     f.data_ptr(), i.data_ptr(), f.data_ptr(), None)
    assert call(64, 64) == tern.TERN_OK
    assert call(64, 96) == 1       # not a power of two
    assert call(64, 32) == 1       # below 64
    assert call(64, 8192) == 1     # above 4096
    assert call(16385, 128) == 3   # K beyond TERN_BLOCK_MAX_K
    torch.cuda.synchronize()
