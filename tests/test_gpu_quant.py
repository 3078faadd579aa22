"""Per-token activation quantiser on the GPU against the oracle: codes, scales
and zero points identical (both take every integer decision from the same
correctly rounded fp32 divisions)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import tern  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402


def _tokens(kind, M, K, rng):
    if kind == "normal":
        x = rng.normal(0, 2.5, (M, K))
    elif kind == "positive":
        x = rng.uniform(0.1, 7.0, (M, K))
    elif kind == "negative":
        x = -rng.exponential(3.0, (M, K))
    elif kind == "wide":
        x = rng.normal(0, 1, (M, K)) * 10.0 ** rng.integers(-20, 20, (M, 1))
    elif kind == "steps":
        # values on and halfway between quantisation steps (ties round to even)
        x = (rng.integers(-255, 256, (M, K)) / 2.0) * (4.0 / 255.0)
    else:
        x = np.zeros((M, K))
    return x.astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "positive", "negative", "wide", "steps", "zeros"])
@pytest.mark.parametrize("M,K", [(1, 1), (3, 100), (8, 4096), (5, 12288), (64, 1000)])
def test_quantize_parity(kind, M, K):
    rng = np.random.default_rng([M, K, len(kind)])
    x = _tokens(kind, M, K, rng)
    ldx, ldq = K + 3, K + 9
    xp = np.zeros((M, ldx), np.float32)
    xp[:, :K] = x
    q = torch.full((M, ldq), 55, dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    z = torch.empty(M, dtype=torch.int32, device=DEV)
    tern.tern_quantize_act(to_dev(xp), M, K, ldx, q, ldq, s, z)
    torch.cuda.synchronize()
    rq, rs, rz = oracle.quantize_act(x)
    qh = q.cpu().numpy()
    assert np.array_equal(qh[:, :K], rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(z.cpu().numpy(), rz)
    assert (qh[:, K:] == 55).all()  # columns past K untouched


def test_quantize_then_linear_roundtrip():
    """Quantised activations feed the ternary GEMV: its output equals the
    oracle's on the same (q, s_act, z)."""
    from gpu_util import gpu_pack
    rng = np.random.default_rng(3)
    N, K = 200, 4096
    w = rng.choice(np.array([-1, 0, 1], np.int8), p=[0.2, 0.6, 0.2], size=(N, K))
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    x = rng.normal(0, 1, (1, K)).astype(np.float32)
    q = torch.empty((1, K), dtype=torch.int8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    z = torch.empty(1, dtype=torch.int32, device=DEV)
    tern.tern_quantize_act(to_dev(x), 1, K, K, q, K, s, z)
    packed, rowsum, _ = gpu_pack(w)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    tern.tern_gemv(packed, to_dev(s_row), rowsum, N, K, q, s, z, y)
    torch.cuda.synchronize()
    rq, rs, rz = oracle.quantize_act(x)
    rp, rr, _ = oracle.pack(w)
    _, ry32, _ = oracle.linear(rp, s_row, rr, K, rq, rs, rz)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ry32[0].view(np.uint32))
