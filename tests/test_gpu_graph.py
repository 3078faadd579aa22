"""A decode step captured in a HIP graph: activation quantiser -> stack of
ternary linears -> int8 head, replayed with new activations between eager
work and synchronisations; every replay must equal the eager run bit for
bit (the calls enqueue kernels only: no allocation, copy or memset).  The
same step with the quantiser fused into the stack launch (two launches)
gives the same bits as the three-launch step."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from packed_bit_gemv_tern_amd import synth, tern  # noqa: E402
from packed_bit_gemv_tern_amd.stack import DeviceStack  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402


@pytest.mark.parametrize("M", [1, 8])
def test_decode_step_graph_replays(M):
    st = DeviceStack("8b", layers=1, seed=11, threads=8)
    b = st.bind(M)
    K = st.linears[0].K
    ldq = b.q[0].shape[1]
    # the head: 2,000 rows of the int8 output head shape
    Wh, srh = synth.make_head(3, 2000, K)
    Whd, srhd = to_dev(Wh), to_dev(srh)
    rsh = torch.empty(2000, dtype=torch.int32, device=DEV)
    tern.tern_head_rowsum(Whd, 2000, K, K, rsh)
    x = torch.empty((M, K), dtype=torch.float32, device=DEV)
    logits = torch.empty((M, 2000), dtype=torch.float32, device=DEV)

    def step():
        # linear 0 of the stack and the head read the freshly quantised tokens
        tern.tern_quantize_act(x, M, K, K, b.q[0], ldq, b.s_act[0], b.z[0])
        b.run()
        tern.tern_head_gemv(Whd, srhd, rsh, 2000, K, K, M, b.q[0], ldq, b.s_act[0], b.z[0], logits, 2000)

    def outputs():
        return [y.clone() for y in b.y] + [logits.clone(), b.q[0].clone()]

    rng = np.random.default_rng(M)
    xs = [rng.normal(0, 1 + i, (M, K)).astype(np.float32) for i in range(4)]
    eager = []
    for xi in xs:
        x.copy_(torch.from_numpy(xi))
        step()
        torch.cuda.synchronize()
        eager.append(outputs())

    g = torch.cuda.CUDAGraph()
    x.copy_(torch.from_numpy(xs[0]))
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(torch.from_numpy(xi))
            for y in b.y:
                y.fill_(float("nan"))  # eager work between replays
            logits.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, e in zip(outputs(), eager[i]):
                assert torch.equal(a.view(torch.uint8), e.view(torch.uint8)), (M, rep, i)


@pytest.mark.parametrize("M", [1, 8])
def test_fused_decode_step_graph_replays(M):
    # layer 0's q/k/v read one fp32 token row that the stack launch quantises
    # itself; the head reads the quantised row after it: two launches
    st = DeviceStack("8b", layers=1, seed=12, threads=8)
    fused = st.bind(M, share_inputs=True, quantise="first")
    sep = st.bind(M, share_inputs=True)
    K = st.linears[0].K
    ldq = sep.q[0].shape[1]
    Wh, srh = synth.make_head(4, 2000, K)
    Whd, srhd = to_dev(Wh), to_dev(srh)
    rsh = torch.empty(2000, dtype=torch.int32, device=DEV)
    tern.tern_head_rowsum(Whd, 2000, K, K, rsh)
    x = fused.x[0]
    assert x is not None and fused.x[1] is x and fused.x[2] is x and fused.x[3] is None
    lf = torch.empty((M, 2000), dtype=torch.float32, device=DEV)
    ls = torch.empty((M, 2000), dtype=torch.float32, device=DEV)

    def step_fused():
        fused.run()
        tern.tern_head_gemv(Whd, srhd, rsh, 2000, K, K, M, fused.q[0], ldq, fused.s_act[0], fused.z[0], lf, 2000)

    def step_sep():
        tern.tern_quantize_act(x, M, K, K, sep.q[0], ldq, sep.s_act[0], sep.z[0])
        sep.run()
        tern.tern_head_gemv(Whd, srhd, rsh, 2000, K, K, M, sep.q[0], ldq, sep.s_act[0], sep.z[0], ls, 2000)

    rng = np.random.default_rng(M + 100)
    xs = [rng.normal(0, 1 + i, (M, K)).astype(np.float32) for i in range(4)]
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step_fused()
    torch.cuda.synchronize()
    for rep in range(2):
        for xi in xs:
            x.copy_(torch.from_numpy(xi))
            for y in fused.y:
                y.fill_(float("nan"))
            lf.zero_()
            torch.cuda.synchronize()
            if rep == 0:
                step_fused()
            else:
                g.replay()
            step_sep()
            torch.cuda.synchronize()
            for a, b_ in zip(fused.y + [lf, fused.q[0], fused.s_act[0], fused.z[0]],
                             sep.y + [ls, sep.q[0], sep.s_act[0], sep.z[0]]):
                assert torch.equal(a.view(torch.int8) if a.dtype != torch.int8 else a,
                                   b_.view(torch.int8) if b_.dtype != torch.int8 else b_), (M, rep)
    tern.tern_linear_stack_status(fused.plan)
