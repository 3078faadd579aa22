"""The int8 output head on the GPU against the oracle: bit-exact acc and fp32
logits (same three roundings), on ragged shapes, padded strides and M = 1..8,
and on sampled rows of the full 151,936 x 4,096 head."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import synth, tern  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402


def _case(N, K, M, seed, ldw_extra=0, ldq_extra=0):
    rng = np.random.default_rng([seed, N, K, M])
    W = rng.integers(-128, 128, (N, K), dtype=np.int8)
    s_row = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    s_act = rng.uniform(0.01, 0.05, M).astype(np.float32)
    z = rng.integers(-128, 129, M).astype(np.int32)
    ldw = (K + 15) // 16 * 16 + 16 * ldw_extra
    ldq = (K + 15) // 16 * 16 + 16 * ldq_extra
    Wp = np.full((N, ldw), 77, np.int8)   # padding columns hold junk
    Wp[:, :K] = W
    qp = np.full((M, ldq), -99, np.int8)
    qp[:, :K] = q
    return W, Wp, ldw, s_row, q, qp, ldq, s_act, z


def _run(Wp, ldw, s_row, N, K, M, qp, ldq, s_act, z, ldy_extra=3):
    Wd = to_dev(Wp)
    rs = torch.empty(N, dtype=torch.int32, device=DEV)
    tern.tern_head_rowsum(Wd, N, K, ldw, rs)
    ldy = N + ldy_extra
    y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((M, ldy), -7, dtype=torch.int32, device=DEV)
    tern.tern_head_gemv(Wd, to_dev(s_row), rs, N, K, ldw, M, to_dev(qp), ldq, to_dev(s_act),
                        to_dev(z), y, ldy, acc)
    torch.cuda.synchronize()
    return rs.cpu().numpy(), y.cpu().numpy(), acc.cpu().numpy()


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("K", [1, 15, 16, 100, 1024, 1040, 4096, 4100])
def test_head_parity(M, K):
    N = 300 if K <= 1040 else 77
    W, Wp, ldw, s_row, q, qp, ldq, s_act, z = _case(N, K, M, seed=1, ldw_extra=1, ldq_extra=1)
    rs, y, acc = _run(Wp, ldw, s_row, N, K, M, qp, ldq, s_act, z)
    rrs = oracle.head_rowsum(W)
    assert np.array_equal(rs, rrs)
    racc, ry32, _ = oracle.head(W, s_row, rrs, q, s_act, z)
    assert np.array_equal(acc[:, :N], racc), (M, K)
    assert np.array_equal(y[:, :N].view(np.uint32), ry32.view(np.uint32)), (M, K)
    # columns past N of each output row are untouched
    assert np.isnan(y[:, N:]).all() and (acc[:, N:] == -7).all()


@pytest.mark.parametrize("N", [1, 5, 31, 33, 1000])
def test_head_ragged_rows(N):
    M, K = 2, 256
    W, Wp, ldw, s_row, q, qp, ldq, s_act, z = _case(N, K, M, seed=2)
    rs, y, acc = _run(Wp, ldw, s_row, N, K, M, qp, ldq, s_act, z, ldy_extra=0)
    racc, ry32, _ = oracle.head(W, s_row, oracle.head_rowsum(W), q, s_act, z)
    assert np.array_equal(acc, racc)
    assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32))


def test_head_errors():
    W = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    f = torch.zeros(16, dtype=torch.float32, device=DEV)
    i = torch.zeros(16, dtype=torch.int32, device=DEV)
    q = torch.zeros((16, 64), dtype=torch.int8, device=DEV)
    y = torch.zeros((16, 8), dtype=torch.float32, device=DEV)
    lib = tern.library()
    args = lambda **kw: dict(dict(W=W, N=8, K=64, ldw=64, M=1, q=q, ldq=64, y=y, ldy=8), **kw)

    def call(a):
        return lib.tern_head_gemv(a["W"].data_ptr(), f.data_ptr(), i.data_ptr(), a["N"], a["K"],
                                  a["ldw"], a["M"], a["q"].data_ptr(), a["ldq"], f.data_ptr(),
                                  i.data_ptr(), a["y"].data_ptr(), a["ldy"], None, None)
    assert call(args()) == tern.TERN_OK
    assert call(args(M=9)) == 4          # TERN_ERR_UNSUPPORTED
    assert call(args(K=43804, ldw=43808)) == 3   # TERN_ERR_RANGE
    assert call(args(ldw=48)) == 1      # ldw < K
    assert call(args(ldw=72, K=64)) == 2  # ldw not a multiple of 16
    assert call(args(M=2, ldq=40)) == 1  # ldq < K
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def head8b():
    W, s_row = synth.make_head(0)
    Wd = to_dev(W)
    N, K = W.shape
    rs = torch.empty(N, dtype=torch.int32, device=DEV)
    tern.tern_head_rowsum(Wd, N, K, K, rs)
    yield W, s_row, Wd, rs
    del Wd
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M", [1, 8])
def test_head_8b_sampled(head8b, M):
    """The full 151,936 x 4,096 head: 512 sampled rows (first and last included)
    against the oracle, bit for bit."""
    W, s_row, Wd, rs = head8b
    N, K = W.shape
    rng = np.random.default_rng([7, M])
    q = rng.integers(-128, 128, (M, K), dtype=np.int8)
    s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
    z = rng.integers(-8, 9, M).astype(np.int32)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tern.tern_head_gemv(Wd, to_dev(s_row), rs, N, K, K, M, to_dev(q), K, to_dev(s_act), to_dev(z),
                        y, N, acc)
    tern.tern_head_gemv(Wd, to_dev(s_row), rs, N, K, K, M, to_dev(q), K, to_dev(s_act), to_dev(z),
                        y, N, acc)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 510, replace=False)]))
    Ws = W[rows]
    rrs = oracle.head_rowsum(Ws)
    assert np.array_equal(rs.cpu().numpy()[rows], rrs)
    racc, ry32, _ = oracle.head(Ws, s_row[rows], rrs, q, s_act, z)
    assert np.array_equal(acc.cpu().numpy()[:, rows], racc)
    assert np.array_equal(y.cpu().numpy()[:, rows].view(np.uint32), ry32.view(np.uint32))
