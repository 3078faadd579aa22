"""Block-wise scales inside the stack launch (the hot path): stacks whose
linears carry one fp32 scale and int32 row sum per block of B columns.  y
must equal the oracle's fp32 evaluation (blocks summed in order from +0, one
rounding per product and per sum) bit for bit, and acc (when asked for) the
exact sum of the block accumulators, sum_j w_ij q_j - z * sum_b rowsum_b."""
import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth, tern

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import DEV, RTOL, gpu_pack, pad_cols, to_dev  # noqa: E402


class BlockedLinear:
    """One block-scaled linear on the device (weights packed there, block
    row sums by tern_block_rowsum) and its oracle results."""

    def __init__(self, seed, N, K, B, M, with_acc):
        self.N, self.K, self.B, self.M = N, K, B, M
        lin = synth.make_linear(seed, 0, 1, N, K, 0.626, M)
        self.lin = lin
        self.s_b = synth.make_block_scales(seed, 0, 1, N, K, B)
        self.packed, _, _ = gpu_pack(lin.w)
        nb = self.s_b.shape[1]
        self.rb = torch.empty((N, nb), dtype=torch.int32, device=DEV)
        tern.tern_block_rowsum(self.packed, N, K, B, self.rb)
        self.s_bd = to_dev(self.s_b)
        qp = pad_cols(lin.q)
        self.ldq = qp.shape[1]
        self.q, self.s_act, self.z = to_dev(qp), to_dev(lin.s_act), to_dev(lin.z)
        self.y = torch.full((M, N + 2), float("nan"), dtype=torch.float32, device=DEV)
        self.acc = torch.full((M, N + 2), -7, dtype=torch.int32, device=DEV) if with_acc else None

    def desc(self):
        return tern.make_desc(self.packed, None, None, self.N, self.K, self.q, self.ldq, self.s_act, self.z,
                              self.y, self.N + 2, self.acc, self.B, self.s_bd, self.rb)

    def check(self, ctx):
        torch.cuda.synchronize()
        lin = self.lin
        rp, rr, _ = oracle.pack(lin.w)
        rb = oracle.block_rowsum(lin.w, self.B)
        assert np.array_equal(self.rb.cpu().numpy(), rb), ctx
        y32, y64, _ = oracle.linear_blocked(rp, self.s_b, rb, self.K, self.B, lin.q, lin.s_act, lin.z)
        y = self.y.cpu().numpy()
        assert np.all(np.isnan(y[:, self.N:])), ctx  # nothing written past N
        y = y[:, :self.N]
        assert np.array_equal(y.view(np.uint32), y32.view(np.uint32)), ctx
        if self.acc is not None:
            # sum_b acc_b: the per-row accumulator with rowsum = sum_b rowsum_b
            racc, _, _ = oracle.linear(rp, np.ones(self.N, np.float32), rb.sum(axis=1).astype(np.int32), self.K,
                                       lin.q, lin.s_act, lin.z, check=False)
            assert np.array_equal(self.acc.cpu().numpy()[:, :self.N], racc), ctx


def _stack(items, M, path=tern.TERN_PATH_AUTO):
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(items), M), dtype=torch.uint8, device=DEV)
    descs = [it.desc() for it in items]
    plan = tern.tern_linear_stack_prepare(descs, M, ws, path)
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)  # twice: the second launch repeats the first's results
    return plan


@pytest.mark.parametrize("B", [64, 128, 256, 512, 1024, 4096])
def test_blocked_stack_m1(B):
    specs = [(300, 4096), (77, 12288), (129, 1024), (64, 2048), (33, 3072), (50, 512), (40, 8192), (17, 16384)]
    items = [BlockedLinear(100 + i, N, K, B, 1, with_acc=(i % 2 == 0)) for i, (N, K) in enumerate(specs)]
    plan = _stack(items, 1)
    assert plan.kernel >= 8 and plan.kernel < 12  # the block-scaled M = 1 kernels
    for it in items:
        it.check("M=1 B=%d K=%d N=%d" % (B, it.K, it.N))


def test_blocked_stack_mixed_with_per_row_linears():
    # block-scaled linears beside per-row ones in one M = 1 launch
    M = 1
    items = [BlockedLinear(7, 500, 4096, 128, M, True), BlockedLinear(8, 200, 12288, 512, M, False)]
    lin = synth.make_linear(9, 0, 2, 300, 4096, 0.626, M)
    packed, rowsum, _ = gpu_pack(lin.w)
    y = torch.empty((M, 300), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, 300), dtype=torch.int32, device=DEV)
    q = to_dev(pad_cols(lin.q))
    keep = (packed, rowsum, q)
    d = tern.make_desc(packed, to_dev(lin.s_row), rowsum, 300, 4096, q, q.shape[1], to_dev(lin.s_act),
                       to_dev(lin.z), y, 300, acc)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(3, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([items[0].desc(), d, items[1].desc()], M, ws)
    tern.tern_linear_stack(plan)
    for it in items:
        it.check("mixed")
    rp, rr, _ = oracle.pack(lin.w)
    racc, ry32, _ = oracle.linear(rp, lin.s_row, rr, 4096, lin.q, lin.s_act, lin.z)
    assert np.array_equal(acc.cpu().numpy(), racc)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ry32.view(np.uint32))
    del keep


@pytest.mark.parametrize("B", [512, 1024, 2048, 4096])
@pytest.mark.parametrize("M", [2, 5, 8, 12, 16])
def test_blocked_stack_mfma(M, B):
    # the activation-window kernels (8 and 16 tokens): blocks of whole
    # 512-column steps; y-only linears of several windows walk window-major
    # (K = 512 and 4,608: units whose last block group is one K-step)
    specs = [(300, 4096), (77, 12288), (129, 1536), (64, 2048), (40, 8192), (33, 16384), (1000, 12288),
             (45, 512), (38, 4608)]
    items = [BlockedLinear(200 + i, N, K, B, M, with_acc=(i % 3 == 1)) for i, (N, K) in enumerate(specs)]
    plan = _stack(items, M)
    assert plan.kernel in (16 + 12, 16 + 13)  # the block-scaled window kernels
    for it in items:
        it.check("M=%d B=%d K=%d N=%d" % (M, B, it.K, it.N))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M", [4, 8])
def test_blocked_stack_mfma_window_major_groups(M):
    # a few multi-window units per workgroup, y only: window-major groups
    # carry the running block sums between passes in the held slots
    specs = [(65536, 8192, 512), (24576, 12288, 1024), (8192, 8192, 2048), (8192, 16384, 4096)]
    items = [BlockedLinear(300 + i, N, K, B, M, with_acc=False) for i, (N, K, B) in enumerate(specs)]
    plan = _stack(items, M)
    assert plan.kernel == 16 + 12
    for it in items:
        it.check("window-major M=%d B=%d K=%d" % (M, it.B, it.K))


@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("M", [2, 3, 5, 8])
def test_blocked_stack_small_blocks_token_by_token(M, B):
    # blocks below 512 columns at 2..8 tokens: the automatic path runs the
    # stack token by token through the one-token kernels
    specs = [(300, 4096), (77, 12288), (129, 1024), (64, 2048), (33, 3072), (50, 512), (40, 8192), (17, 16384)]
    items = [BlockedLinear(400 + i, N, K, B, M, with_acc=(i % 2 == 0)) for i, (N, K) in enumerate(specs)]
    plan = _stack(items, M)
    assert 12 <= plan.kernel < 16  # the token-by-token kernels
    for it in items:
        it.check("tokens M=%d B=%d K=%d N=%d" % (M, B, it.K, it.N))


@pytest.mark.parametrize("M", [2, 6])
def test_blocked_stack_token_by_token_with_per_row_linears(M):
    # per-row linears (one of ragged K) beside block-scaled ones, token by token
    items = [BlockedLinear(17, 500, 4096, 128, M, True), BlockedLinear(18, 200, 12288, 512, M, False)]
    rows = []
    for i, (N, K) in enumerate([(300, 4096), (90, 100), (64, 12288)]):
        lin = synth.make_linear(19 + i, 0, 2, N, K, 0.626, M)
        packed, rowsum, _ = gpu_pack(lin.w)
        q = to_dev(pad_cols(lin.q))
        y = torch.full((M, N + 1), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((M, N + 1), dtype=torch.int32, device=DEV) if i != 1 else None
        bufs = (packed, rowsum, q, to_dev(lin.s_row), to_dev(lin.s_act), to_dev(lin.z), y, acc)
        rows.append((lin, bufs, tern.make_desc(packed, bufs[3], rowsum, N, K, q, q.shape[1], bufs[4], bufs[5],
                                               y, N + 1, acc)))
    descs = [items[0].desc(), rows[0][2], rows[1][2], items[1].desc(), rows[2][2]]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(descs), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare(descs, M, ws)
    assert 12 <= plan.kernel < 16
    tern.tern_linear_stack(plan)
    for it in items:
        it.check("mixed tokens M=%d" % M)
    for lin, bufs, _ in rows:
        rp, rr, _ = oracle.pack(lin.w)
        racc, ry32, _ = oracle.linear(rp, lin.s_row, rr, lin.K, lin.q, lin.s_act, lin.z)
        y = bufs[6].cpu().numpy()
        assert np.all(np.isnan(y[:, lin.N:]))
        assert np.array_equal(y[:, :lin.N].view(np.uint32), ry32.view(np.uint32)), (M, lin.N, lin.K)
        if bufs[7] is not None:
            assert np.array_equal(bufs[7].cpu().numpy()[:, :lin.N], racc), (M, lin.N, lin.K)


def test_blocked_stack_rejections():
    # block sizes the stack cannot take come back as errors before any launch
    M = 8
    it = BlockedLinear(3, 64, 4096, 512, M, False)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=DEV)
    d = it.desc()
    d.block = 128  # the MFMA path takes whole 512-column steps
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d], M, ws, tern.TERN_PATH_MFMA)
    assert e.value.status == tern.TERN_ERR_UNSUPPORTED
    # ... and the vector ALU at most TERN_VALU_MAX_M tokens
    it12 = BlockedLinear(4, 64, 4096, 512, 12, False)
    ws12 = torch.empty(tern.tern_linear_stack_workspace_bytes(1, 12), dtype=torch.uint8, device=DEV)
    d12 = it12.desc()
    d12.block = 128
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d12], 12, ws12)
    assert e.value.status == tern.TERN_ERR_UNSUPPORTED
    d.block = 96
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d], M, ws)
    assert e.value.status == tern.TERN_ERR_INVALID_ARG
    d.block = 128
    d.s_block = None
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d], M, ws)
    assert e.value.status == tern.TERN_ERR_INVALID_ARG
