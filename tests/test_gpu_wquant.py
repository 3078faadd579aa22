"""The weight quantiser on the GPU against the oracle: states and block
scales bit-exact (fp64 block sums in column order, correctly rounded
divisions, half-to-even rounding), on ragged blocks, strided rows, ties and
zero blocks; and the chain quantise -> pack -> block row sums -> block-scaled
GEMV against the oracle's chain."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import synth, tern  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402


def _gpu_quantize(W, B, ldw_extra=0, ldt_extra=0):
    N, K = W.shape
    ldw, ldt = K + ldw_extra, K + ldt_extra
    Wp = np.full((N, ldw), np.float32(1e30), np.float32)  # junk past K
    Wp[:, :K] = W
    nb = -(-K // B)
    t = torch.full((N, ldt), 77, dtype=torch.int8, device=DEV)
    s = torch.full((N, nb), float("nan"), dtype=torch.float32, device=DEV)
    tern.tern_quantize_weights(to_dev(Wp), N, K, ldw, B, t, ldt, s)
    torch.cuda.synchronize()
    t = t.cpu().numpy()
    assert (t[:, K:] == 77).all()  # nothing written past K
    return t[:, :K], s.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 64, 128, 1000, 5000])
@pytest.mark.parametrize("K", [1, 5, 100, 4096, 4100])
def test_wquant_parity(K, B):
    rng = np.random.default_rng([K, B])
    N = 37
    W = (rng.standard_normal((N, K)) * rng.uniform(1e-3, 10, (N, 1))).astype(np.float32)
    W[3] = 0.0                      # an all-zero row: zero blocks
    W[4, : min(K, B)] = 0.0         # one zero block
    t, s = _gpu_quantize(W, B, ldw_extra=3, ldt_extra=5)
    rt, rs = oracle.quantize_weights(W, B)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), (K, B)
    assert np.array_equal(t, rt), (K, B)


def test_wquant_ties_and_clamps():
    # blocks of two whose mean is exactly 1: ratios of exactly +-0.5 and
    # +-1.5; and blocks whose ratios pass +-1
    W = np.array([[0.5, 1.5, -0.5, -1.5, 0.25, 1.75, 3.0, 1.0]], np.float32)
    t, s = _gpu_quantize(W, 2)
    rt, rs = oracle.quantize_weights(W, 2)
    assert np.array_equal(t, rt) and np.array_equal(s, rs)
    assert t.tolist() == [[0, 1, 0, -1, 0, 1, 1, 0]]


def test_wquant_8b_gate_shape():
    layer, idx = 1, 4
    N, K = 12288, 4096
    rng = np.random.default_rng([layer, idx, 7])
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    t, s = _gpu_quantize(W, 128)
    rows = np.arange(0, N, 97)
    rt, rs = oracle.quantize_weights(W[rows], 128)
    assert np.array_equal(t[rows], rt) and np.array_equal(s[rows].view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("B", [64, 128, 1024])
def test_quantise_pack_blocked_gemv_chain(B):
    rng = np.random.default_rng(B)
    N, K = 300, 4096
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    t, s = _gpu_quantize(W, B)
    # device chain: pack the states, block row sums, block-scaled GEMV
    td = to_dev(np.ascontiguousarray(t))
    packed = torch.empty((N, tern.tern_row_bytes(K)), dtype=torch.uint8, device=DEV)
    rsum = torch.empty(N, dtype=torch.int32, device=DEV)
    tern.tern_pack(td, N, K, K, packed, rsum)
    nb = K // B
    rb = torch.empty((N, nb), dtype=torch.int32, device=DEV)
    tern.tern_block_rowsum(packed, N, K, B, rb)
    q, s_act, z = synth.make_activations(3, 0, 0, K, 1)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    tern.tern_gemv_blocked(packed, to_dev(s), rb, N, K, B, to_dev(q.reshape(-1)), to_dev(s_act), to_dev(z), y)
    torch.cuda.synchronize()
    # oracle chain from the fp32 weights
    rt, rsc = oracle.quantize_weights(W, B)
    opk, _, bad = oracle.pack(rt)
    assert bad == 0
    assert np.array_equal(packed.cpu().numpy(), opk)
    orb = oracle.block_rowsum(rt, B)
    assert np.array_equal(rb.cpu().numpy(), orb)
    _, y64, yabs = oracle.linear_blocked(opk, rsc, orb, K, B, q, s_act, z)
    tol = (nb + 1) * 2.0 ** -24 * yabs[0] * 1.001 + 1e-30
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - y64[0]) <= tol)
