"""The activation quantiser fused into the stack launch.

A linear that names an fp32 input x has its q, s_act and z written by the
launch itself, each distinct q buffer once, before any linear reads them.
Those must equal oracle.quantize_act(x) bit for bit (columns past K of q
untouched), and every output the oracle's linear on them: on every kernel
of the stack (VALU at M = 1 and 2..8, the activation-window kernels with and
without the split along K, the lockstep kernel of ragged K, the prefill
GEMM, block scales), over several launches of one plan whose fp32 inputs
change in between (each launch numbers its flags afresh), from a HIP graph,
and from the library's static workspace."""
import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth, tern

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import DEV, RTOL, gpu_pack, to_dev  # noqa: E402

FILL = 77  # q bytes past K: the launch never writes them


class Input:
    """One activation buffer: an fp32 input the launch quantises, or the
    caller's int8 activations."""

    def __init__(self, seed, idx, K, M, fused):
        self.K, self.M, self.fused, self.seed, self.idx = K, M, fused, seed, idx
        self.ldq = K if M == 1 else (K + 15) // 16 * 16 + 16
        self.ldx = K + 5
        if fused:
            self.q = torch.full((M, self.ldq), FILL, dtype=torch.int8, device=DEV)
            self.s_act = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
            self.z = torch.full((M,), -999, dtype=torch.int32, device=DEV)
            self.xd = torch.zeros((M, self.ldx), dtype=torch.float32, device=DEV)
            self.refill(0)
        else:
            q, s_act, z = synth.make_activations(seed, 0, idx, K, M)
            qp = np.full((M, self.ldq), FILL, np.int8)
            qp[:, :K] = q
            self.q, self.s_act, self.z = to_dev(qp), to_dev(s_act), to_dev(z)
            self.ref = (q, s_act, z)
            self.xd = None

    def refill(self, n):
        """New fp32 values (launch n), written into the same device buffer."""
        x = synth.make_hidden(self.seed + 1000 * n, 0, self.idx, self.K, self.M)
        if n % 3 == 2:
            x[0] = 0.0  # an all-zero token: s_act = 1, z = -128
        self.x = x
        xp = np.zeros((self.M, self.ldx), np.float32)
        xp[:, : self.K] = x
        self.xd.copy_(torch.from_numpy(xp))
        self.ref = oracle.quantize_act(x)

    def check(self, ctx):
        q = self.q.cpu().numpy()
        rq, rs, rz = self.ref
        assert np.array_equal(q[:, : self.K], rq), ctx
        assert np.all(q[:, self.K:] == FILL), ctx
        assert np.array_equal(self.s_act.cpu().numpy().view(np.uint32), rs.view(np.uint32)), ctx
        assert np.array_equal(self.z.cpu().numpy(), rz), ctx


class Lin:
    """One linear reading `inp`; names x when `names_x` (otherwise it only
    reads the buffer another linear's x fills)."""

    def __init__(self, seed, idx, N, K, M, inp, names_x, with_acc, block=0):
        self.N, self.K, self.M, self.inp, self.block = N, K, M, inp, block
        self.names_x = names_x and inp.fused
        lin = synth.make_linear(seed, 0, idx, N, K, 0.626, M)
        self.w, self.s_row = lin.w, lin.s_row
        self.packed, self.rowsum, _ = gpu_pack(lin.w)
        self.s_rowd = to_dev(lin.s_row)
        if block:
            self.s_b = synth.make_block_scales(seed, 0, idx, N, K, block)
            self.s_bd = to_dev(self.s_b)
            self.rb = torch.empty((N, self.s_b.shape[1]), dtype=torch.int32, device=DEV)
            tern.tern_block_rowsum(self.packed, N, K, block, self.rb)
        self.y = torch.full((M, N + 1), float("nan"), dtype=torch.float32, device=DEV)
        self.acc = torch.full((M, N + 1), -7, dtype=torch.int32, device=DEV) if with_acc else None
        if N > 0:
            self.rp, self.rr, _ = oracle.pack(lin.w)

    def desc(self):
        i = self.inp
        kw = dict(x=i.xd, ldx=i.ldx) if self.names_x else {}
        if self.block:
            return tern.make_desc(self.packed, None, None, self.N, self.K, i.q, i.ldq, i.s_act, i.z, self.y,
                                  self.N + 1, self.acc, self.block, self.s_bd, self.rb, **kw)
        return tern.make_desc(self.packed, self.s_rowd, self.rowsum, self.N, self.K, i.q, i.ldq, i.s_act, i.z,
                              self.y, self.N + 1, self.acc, **kw)

    def check(self, ctx):
        q, s_act, z = self.inp.ref
        y = self.y.cpu().numpy()
        assert np.all(np.isnan(y[:, self.N:])), ctx
        y = y[:, : self.N]
        if self.block:
            rb = oracle.block_rowsum(self.w, self.block)
            ry32, _, _ = oracle.linear_blocked(self.rp, self.s_b, rb, self.K, self.block, q, s_act, z)
            assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), ctx
            return
        racc, ry32, ry64 = oracle.linear(self.rp, self.s_row, self.rr, self.K, q, s_act, z)
        if self.acc is not None:
            assert np.array_equal(self.acc.cpu().numpy()[:, : self.N], racc), ctx
        assert np.all(np.abs(y.astype(np.float64) - ry64) <= RTOL * np.abs(ry64)), ctx
        assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), ctx


# (N, K, input group, names x); group -1: the linear's own caller activations
SPECS = [(300, 4096, 0, True), (129, 4096, 0, False), (77, 12288, 1, True), (64, 2048, -1, False),
         (500, 1024, 2, True), (33, 4096, 0, True), (96, 12288, 1, False)]


def build(M, specs, seed, block=0, with_acc=True):
    inputs, lins = {}, []
    for i, (N, K, g, nx) in enumerate(specs):
        key = g if g >= 0 else ("own", i)
        if key not in inputs:
            inputs[key] = Input(seed + 17 * i, i, K, M, fused=g >= 0)
        lins.append(Lin(seed, i, N, K, M, inputs[key], nx, with_acc and i % 2 == 0, block))
    return list(inputs.values()), lins


def run_launches(inputs, lins, M, path, launches=3, static=False):
    descs = [l.desc() for l in lins]
    if static:
        plan = tern.tern_linear_stack_prepare_static(descs, M, path)
        ws = None
    else:
        ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(descs), M), dtype=torch.uint8, device=DEV)
        plan = tern.tern_linear_stack_prepare(descs, M, ws, path)
    for n in range(launches):
        if n > 0:
            for i in inputs:
                if i.fused:
                    i.refill(n)
        tern.tern_linear_stack(plan)
        torch.cuda.synchronize()
        for i in inputs:
            i.check("launch %d input %d" % (n, i.idx))
        for k, l in enumerate(lins):
            l.check("launch %d linear %d (N=%d K=%d M=%d)" % (n, k, l.N, l.K, M))
    tern.tern_linear_stack_status(plan)
    del ws
    return plan


CASES = [
    # name, M, path, extra specs, kernel selector check
    ("valu_m1", 1, tern.TERN_PATH_AUTO, [], lambda k: k < 8),
    ("valu_m4", 4, tern.TERN_PATH_VALU, [], lambda k: 4 <= k <= 6),
    ("window_m5_split", 5, tern.TERN_PATH_AUTO, [], lambda k: k == 16 + 8),
    ("window_m8_split", 8, tern.TERN_PATH_AUTO, [], lambda k: k == 16 + 8),
    ("lockstep_ragged_m3", 3, tern.TERN_PATH_AUTO, [(200, 1000, 3, True), (70, 1000, 3, False)],
     lambda k: k == 16 + 2),
    ("gemm_m12", 12, tern.TERN_PATH_AUTO, [], lambda k: k in (16 + 9, 16 + 10)),
    ("gemm_m64", 64, tern.TERN_PATH_AUTO, [], lambda k: k == 16 + 9),
    ("gemm_m200", 200, tern.TERN_PATH_AUTO, [], lambda k: k == 16 + 14),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,M,path,extra,kcheck", CASES, ids=[c[0] for c in CASES])
def test_fused_quantiser_every_kernel(name, M, path, extra, kcheck):
    inputs, lins = build(M, SPECS + extra, seed=40 + M)
    plan = run_launches(inputs, lins, M, path)
    assert kcheck(plan.kernel), (name, plan.kernel)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("M,B", [(1, 128), (1, 1024), (8, 512), (16, 1024), (4, 128), (8, 256)])
def test_fused_quantiser_block_scales(M, B):
    specs = [(300, 4096, 0, True), (129, 4096, 0, False), (77, 12288, 1, True), (64, 2048, -1, False),
             (40, 8192, 2, True)]
    inputs, lins = build(M, specs, seed=70 + M, block=B, with_acc=False)
    plan = run_launches(inputs, lins, M, tern.TERN_PATH_AUTO)
    if M == 1:
        assert plan.kernel in (8, 9, 10, 11)
    elif B % 512:
        assert plan.kernel in (12, 13, 14, 15)  # token by token on the vector ALU
    else:
        assert plan.kernel in (16 + 12, 16 + 13)


@pytest.mark.timeout(300)
def test_fused_quantiser_window_kernels_deep_stack():
    # stacks deep enough for the unsplit 8- and 16-token window kernels, with
    # held outputs and window-major linears (K = 12,288, y only)
    specs = [(2048, 4096, i % 5, True) for i in range(40)] + [(1024, 12288, 5, True), (1024, 12288, 5, True)]
    for M, kern in ((8, 16 + 8), (16, 16 + 11)):
        inputs, lins = build(M, specs, seed=90 + M, with_acc=False)
        # each group's first linear names x (the others read its q)
        seen = set()
        for l in lins:
            l.names_x = l.inp.fused and id(l.inp) not in seen
            seen.add(id(l.inp))
        plan = run_launches(inputs, lins, M, tern.TERN_PATH_AUTO, launches=2)
        assert plan.kernel == kern and plan.splits == 0, (M, plan.kernel, plan.splits)


def test_fused_quantiser_static_workspace():
    M = 8
    inputs, lins = build(M, SPECS, seed=5)
    run_launches(inputs, lins, M, tern.TERN_PATH_AUTO, launches=2, static=True)


def test_fused_quantiser_input_of_a_linear_without_rows():
    # a linear with N = 0 still has its input quantised (q is an output)
    M = 4
    inp = Input(11, 0, 4096, M, fused=True)
    other = Input(12, 1, 2048, M, fused=False)
    empty = Lin(11, 0, 0, 4096, M, inp, True, False)
    full = Lin(12, 1, 100, 2048, M, other, False, True)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(2, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([empty.desc(), full.desc()], M, ws)
    tern.tern_linear_stack(plan)
    torch.cuda.synchronize()
    inp.check("N = 0 linear's input")
    full.check("linear beside it")


def test_fused_quantiser_graph_replays():
    # one fused launch captured in a HIP graph and replayed, the fp32 inputs
    # rewritten eagerly between replays: every replay quantises afresh
    M = 8
    inputs, lins = build(M, SPECS, seed=23)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(lins), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([l.desc() for l in lins], M, ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tern.tern_linear_stack(plan, s)  # (eager, on the capture stream, once)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tern.tern_linear_stack(plan, s)
    torch.cuda.synchronize()
    for n in range(1, 5):
        for i in inputs:
            if i.fused:
                i.refill(n)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in inputs:
            i.check("replay %d" % n)
        for l in lins:
            l.check("replay %d N=%d" % (n, l.N))
    tern.tern_linear_stack_status(plan)


def test_fused_quantiser_rejections():
    M = 8
    inputs, lins = build(M, SPECS[:3], seed=3)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(3, M), dtype=torch.uint8, device=DEV)
    descs = [l.desc() for l in lins]
    # a second linear naming the same q with another x
    d = lins[1].desc()
    other = torch.zeros((M, 4096), dtype=torch.float32, device=DEV)
    d.x, d.ldx = other.data_ptr(), 4096
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([descs[0], d, descs[2]], M, ws)
    assert e.value.status == tern.TERN_ERR_INVALID_ARG
    # a reader of a quantised q naming other scales
    d = lins[1].desc()
    d.s_act = inputs[1].s_act.data_ptr()
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([descs[0], d, descs[2]], M, ws)
    assert e.value.status == tern.TERN_ERR_INVALID_ARG
    # x rows shorter than K, misaligned x
    d = lins[0].desc()
    d.ldx = 4095
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d], M, ws)
    assert e.value.status == tern.TERN_ERR_INVALID_ARG
    d = lins[0].desc()
    d.x = d.x + 2
    with pytest.raises(tern.TernError) as e:
        tern.tern_linear_stack_prepare([d], M, ws)
    assert e.value.status == tern.TERN_ERR_ALIGNMENT
