"""The gated feed-forward chained over two launches (model card "Neutrino-1
8B", "Architecture": a gated SwiGLU feed-forward of three linears per layer):
launch 1 quantises the fp32 hidden state and runs gate and up; launch 2
quantises h = silu(g) * u, formed from launch 1's outputs inside its own
prologue, and runs down.  Every intermediate is compared with the oracle
chain: quantise_act -> linear (gate, up) -> swiglu -> quantise_act -> linear
(down), bit for bit (codes, scales, zero points, acc, y), on every stack
kernel (VALU at M = 1, the 8- and 16-token window kernels, the GEMM)."""
import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth, tern

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import DEV, gpu_pack, to_dev  # noqa: E402


def _pad16(n):
    return (n + 15) // 16 * 16


class Lin:
    """A linear on the device with its own output buffers."""

    def __init__(self, seed, idx, N, K, M, p_zero):
        self.w, self.s_row = synth.make_weights(seed, 0, idx, N, K, p_zero)
        self.N, self.K = N, K
        self.packed, self.rowsum, _ = gpu_pack(self.w)
        self.s_rowd = to_dev(self.s_row)
        self.y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        self.acc = torch.full((M, N), -7, dtype=torch.int32, device=DEV)

    def desc(self, q, ldq, s_act, z, **kw):
        return tern.make_desc(self.packed, self.s_rowd, self.rowsum, self.N, self.K, q, ldq, s_act, z,
                              self.y, self.N, self.acc, **kw)

    def oracle(self, q, s_act, z):
        rp, rr, _ = oracle.pack(self.w)
        return oracle.linear(rp, self.s_row, rr, self.K, q, s_act, z)


def _check_quant(qd, sd, zd, K, rq, rs, rz, ctx):
    assert np.array_equal(qd.cpu().numpy()[:, :K], rq), ctx
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), rs.view(np.uint32)), ctx
    assert np.array_equal(zd.cpu().numpy(), rz), ctx


def _check_lin(lin, racc, ry32, ctx):
    assert np.array_equal(lin.acc.cpu().numpy(), racc), ctx
    assert np.array_equal(lin.y.cpu().numpy().view(np.uint32), ry32.view(np.uint32)), ctx


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M", [1, 3, 8, 16, 64])
def test_ffn_chain_two_launches(M):
    # an FFN of reduced width (hidden 1024, FFN 3072: the 0.6B shapes) and one
    # of the 8B's down shape (K = 12,288) beside it
    H, F = 1024, 3072
    x = synth.make_hidden(5, 0, 0, H, M)
    gate, up = Lin(5, 4, F, H, M, 0.7), Lin(5, 5, F, H, M, 0.62)
    down = Lin(5, 6, H, F, M, 0.7)
    ldq1, ldq2 = _pad16(H), _pad16(F)
    xd = to_dev(x)
    q1 = torch.zeros((M, ldq1), dtype=torch.int8, device=DEV)
    s1 = torch.empty(M, dtype=torch.float32, device=DEV)
    z1 = torch.empty(M, dtype=torch.int32, device=DEV)
    q2 = torch.zeros((M, ldq2), dtype=torch.int8, device=DEV)
    s2 = torch.empty(M, dtype=torch.float32, device=DEV)
    z2 = torch.empty(M, dtype=torch.int32, device=DEV)
    # launch 1: quantise x, then gate and up reading it
    d1 = [gate.desc(q1, ldq1, s1, z1, x=xd, ldx=H), up.desc(q1, ldq1, s1, z1, x=xd, ldx=H)]
    ws1 = torch.empty(tern.tern_linear_stack_workspace_bytes(2, M), dtype=torch.uint8, device=DEV)
    p1 = tern.tern_linear_stack_prepare(d1, M, ws1)
    # launch 2: quantise silu(g) * u from launch 1's outputs, then down
    d2 = [down.desc(q2, ldq2, s2, z2, x=gate.y, ldx=F, x_up=up.y)]
    ws2 = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=DEV)
    p2 = tern.tern_linear_stack_prepare(d2, M, ws2)
    for launch in range(2):  # twice: the second pair repeats the first's results
        tern.tern_linear_stack(p1)
        tern.tern_linear_stack(p2)
        torch.cuda.synchronize()
        ctx = "M=%d launch %d kernels %d/%d" % (M, launch, p1.kernel, p2.kernel)
        rq1, rs1, rz1 = oracle.quantize_act(x)
        _check_quant(q1, s1, z1, H, rq1, rs1, rz1, ctx)
        ag, yg, _ = gate.oracle(rq1, rs1, rz1)
        au, yu, _ = up.oracle(rq1, rs1, rz1)
        _check_lin(gate, ag, yg, ctx + " gate")
        _check_lin(up, au, yu, ctx + " up")
        h = oracle.swiglu(yg, yu)
        rq2, rs2, rz2 = oracle.quantize_act(h)
        _check_quant(q2, s2, z2, F, rq2, rs2, rz2, ctx + " h")
        ad, yd, _ = down.oracle(rq2, rs2, rz2)
        _check_lin(down, ad, yd, ctx + " down")


@pytest.mark.parametrize("M", [1, 8])
def test_swiglu_input_8b_down_shape(M):
    # the 8B's down projection (12,288 -> 4,096, rows sampled to 256) reading
    # gate and up outputs with wide ranges, large gates and very negative ones
    K, N = 12288, 256
    rng = np.random.default_rng([7, M])
    g = (rng.normal(0, 4, (M, K)) * (1 + 20 * (rng.random((M, K)) < 0.004))).astype(np.float32)
    g[:, :8] = [0.0, -88.0, -89.0, -1e30, 17.0, 1e4, -0.0, 1e-30]
    u = rng.normal(0, 2, (M, K)).astype(np.float32)
    down = Lin(7, 6, N, K, M, 0.72)
    ldq = _pad16(K)
    q = torch.zeros((M, ldq), dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    z = torch.empty(M, dtype=torch.int32, device=DEV)
    gd, ud = to_dev(g), to_dev(u)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([down.desc(q, ldq, s, z, x=gd, ldx=K, x_up=ud)], M, ws)
    tern.tern_linear_stack(plan)
    torch.cuda.synchronize()
    rq, rs, rz = oracle.quantize_act(oracle.swiglu(g, u))
    _check_quant(q, s, z, K, rq, rs, rz, "M=%d" % M)
    racc, ry32, _ = down.oracle(rq, rs, rz)
    _check_lin(down, racc, ry32, "M=%d" % M)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M", [1, 8])
def test_ffn_chain_graph_replays_static_workspace(M):
    # the two launches captured in a HIP graph, the down launch prepared in the
    # library's static workspace: every replay, with new hidden states and
    # eager launches of the same plans in between, matches the oracle chain
    H, F = 1024, 3072
    gate, up, down = Lin(9, 4, F, H, M, 0.7), Lin(9, 5, F, H, M, 0.62), Lin(9, 6, H, F, M, 0.7)
    ldq1, ldq2 = _pad16(H), _pad16(F)
    xd = torch.empty((M, H), dtype=torch.float32, device=DEV)
    q1 = torch.zeros((M, ldq1), dtype=torch.int8, device=DEV)
    s1 = torch.empty(M, dtype=torch.float32, device=DEV)
    z1 = torch.empty(M, dtype=torch.int32, device=DEV)
    q2 = torch.zeros((M, ldq2), dtype=torch.int8, device=DEV)
    s2 = torch.empty(M, dtype=torch.float32, device=DEV)
    z2 = torch.empty(M, dtype=torch.int32, device=DEV)
    d1 = [gate.desc(q1, ldq1, s1, z1, x=xd, ldx=H), up.desc(q1, ldq1, s1, z1, x=xd, ldx=H)]
    ws1 = torch.empty(tern.tern_linear_stack_workspace_bytes(2, M), dtype=torch.uint8, device=DEV)
    p1 = tern.tern_linear_stack_prepare(d1, M, ws1)
    p2 = tern.tern_linear_stack_prepare_static([down.desc(q2, ldq2, s2, z2, x=gate.y, ldx=F, x_up=up.y)], M)

    def check(x, ctx):
        rq1, rs1, rz1 = oracle.quantize_act(x)
        _, yg, _ = gate.oracle(rq1, rs1, rz1)
        _, yu, _ = up.oracle(rq1, rs1, rz1)
        rq2, rs2, rz2 = oracle.quantize_act(oracle.swiglu(yg, yu))
        _check_quant(q2, s2, z2, F, rq2, rs2, rz2, ctx)
        ad, yd, _ = down.oracle(rq2, rs2, rz2)
        _check_lin(down, ad, yd, ctx)

    rng = np.random.default_rng(M + 300)
    xs = [(rng.normal(0, 1 + i, (M, H)) * (1 + 20 * (rng.random((M, H)) < 0.004))).astype(np.float32)
          for i in range(3)]
    xd.copy_(torch.from_numpy(xs[0]))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        tern.tern_linear_stack(p1)
        tern.tern_linear_stack(p2)
    torch.cuda.synchronize()
    for rep, x in enumerate(xs):
        for eager in (False, True):
            xd.copy_(torch.from_numpy(x))
            down.y.fill_(float("nan"))
            torch.cuda.synchronize()
            if eager:
                tern.tern_linear_stack(p1)
                tern.tern_linear_stack(p2)
            else:
                graph.replay()
            torch.cuda.synchronize()
            check(x, "M=%d input %d %s" % (M, rep, "eager" if eager else "replay"))
