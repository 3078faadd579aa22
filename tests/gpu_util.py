"""Helpers for the GPU parity tests: upload seeded inputs, run the library
through its C ABI, and compare with the oracle on the CPU."""
import numpy as np
import torch

import oracle
from packed_bit_gemv_tern_amd import tern

DEV = "cuda:0"
RTOL = 1e-6  # fp32 outputs against the fp64 oracle value


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def pad_cols(q: np.ndarray, mult: int = 16) -> np.ndarray:
    """Copy an (M, K) int8 activation block into rows of a 16-multiple stride."""
    M, K = q.shape
    ldq = (K + mult - 1) // mult * mult
    out = np.zeros((M, ldq), np.int8)
    out[:, :K] = q
    return out


def gpu_pack(w: np.ndarray):
    """Pack an (N, K) int8 matrix on the GPU -> (packed, rowsum, bad) tensors."""
    N, K = w.shape
    wd = to_dev(w)
    packed = torch.empty((max(N, 1), tern.tern_row_bytes(K)), dtype=torch.uint8, device=DEV)
    rowsum = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    bad = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    tern.tern_pack(wd, N, K, K, packed, rowsum, bad)
    return packed, rowsum, bad


class Uploaded:
    """One linear's inputs on the device, packed by the library."""

    def __init__(self, lin, ldy_extra: int = 0, with_acc: bool = True):
        self.lin = lin
        N, K, M = lin.N, lin.K, lin.M
        self.packed, self.rowsum, self.bad = gpu_pack(lin.w)
        self.s_row = to_dev(lin.s_row)
        qp = pad_cols(lin.q)
        self.ldq = qp.shape[1]
        self.q = to_dev(qp)
        self.s_act = to_dev(lin.s_act.astype(np.float32))
        self.z = to_dev(lin.z.astype(np.int32))
        self.ldy = N + ldy_extra
        self.y = torch.full((M, self.ldy), float("nan"), dtype=torch.float32, device=DEV)
        self.acc = torch.full((M, self.ldy), -7, dtype=torch.int32, device=DEV) if with_acc else None

    def run(self, path=tern.TERN_PATH_AUTO):
        lin = self.lin
        if lin.M == 1 and path == tern.TERN_PATH_AUTO:
            tern.tern_gemv(self.packed, self.s_row, self.rowsum, lin.N, lin.K, self.q, self.s_act,
                           self.z, self.y, self.acc)
        else:
            tern.tern_gemm_smallM(self.packed, self.s_row, self.rowsum, lin.N, lin.K, lin.M, self.q,
                                  self.ldq, self.s_act, self.z, self.y, self.ldy, self.acc, path)

    def desc(self):
        lin = self.lin
        return tern.make_desc(self.packed, self.s_row, self.rowsum, lin.N, lin.K, self.q,
                              self.ldq, self.s_act, self.z, self.y, self.ldy, self.acc)

    def results(self):
        torch.cuda.synchronize()
        N = self.lin.N
        if self.acc is None:
            return self.y.cpu().numpy()[:, :N], None
        return self.y.cpu().numpy()[:, :N], self.acc.cpu().numpy()[:, :N]


def oracle_ref(lin, rows=None):
    """Oracle acc / y32 / y64 of a linear, optionally on a subset of rows."""
    w = lin.w if rows is None else lin.w[rows]
    s_row = lin.s_row if rows is None else lin.s_row[rows]
    packed, rowsum, bad = oracle.pack(w)
    assert bad == 0
    return oracle.linear(packed, s_row, rowsum, lin.K, lin.q, lin.s_act, lin.z)


def assert_parity(y, acc, ref, ctx=""):
    """acc bit-exact; y within RTOL of the fp64 value (zero exactly) and
    bit-identical to the ordered fp32 evaluation."""
    racc, ry32, ry64 = ref
    if acc is not None:  # (y-only calls: no acc to compare)
        bad = np.argwhere(acc != racc)
        assert bad.size == 0, "%s acc mismatch at %s: gpu %s oracle %s" % (
            ctx, bad[:5].tolist(), acc[tuple(bad[0])], racc[tuple(bad[0])])
    err = np.abs(y.astype(np.float64) - ry64)
    lim = RTOL * np.abs(ry64)
    worst = np.argmax(err - lim)
    assert np.all(err <= lim), "%s y outside 1e-6 at %s: %r vs %r" % (
        ctx, np.unravel_index(worst, y.shape), y.flat[worst], ry64.flat[worst])
    assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), "%s y not bit-identical" % ctx
