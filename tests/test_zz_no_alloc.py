"""The allocation-free stack prepare (tern_linear_stack_prepare_static): its
schedule lives in the library's static device workspace.  Its launches must
give the same bits as the workspace-taking prepare's, on two prepares in a
row, the second with a smaller stack (the array keeps the first schedule's
contents, which the second must replace), and meet the oracle."""
import numpy as np
import pytest

from packed_bit_gemv_tern_amd import synth, tern

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import DEV, Uploaded, assert_parity, oracle_ref  # noqa: E402


def _same_as_workspace_prepare(lins, M, with_acc):
    ref = [Uploaded(lin, with_acc=with_acc) for lin in lins]
    got = [Uploaded(lin, with_acc=with_acc) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(lins), M), dtype=torch.uint8, device=DEV)
    plan_ref = tern.tern_linear_stack_prepare([u.desc() for u in ref], M, ws)
    plan = tern.tern_linear_stack_prepare_static([u.desc() for u in got], M)
    assert plan.workspace and plan.workspace != plan_ref.workspace
    assert (plan.kernel, plan.grid, plan.workers, plan.segments) == \
        (plan_ref.kernel, plan_ref.grid, plan_ref.workers, plan_ref.segments)
    tern.tern_linear_stack(plan_ref)
    tern.tern_linear_stack(plan)
    for lin, a, b in zip(lins, ref, got):
        ya, acca = a.results()
        yb, accb = b.results()
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), lin.name
        if with_acc:
            assert np.array_equal(acca, accb), lin.name
        assert_parity(yb, accb, oracle_ref(lin), "static %s M=%d" % (lin.name, M))
    return plan


@pytest.mark.parametrize("M", [1, 8])
def test_static_prepare_two_stacks_in_a_row(M):
    first = synth.make_stack(41, M, model="0.6b", layers=2, threads=8)
    p1 = _same_as_workspace_prepare(first, M, with_acc=True)
    second = synth.make_stack(42, M, model="0.6b", layers=1, threads=8)[:4]
    p2 = _same_as_workspace_prepare(second, M, with_acc=False)
    assert p2.workspace == p1.workspace  # one array per device
    assert p2.segments <= p1.segments


def test_static_prepare_refuses_a_schedule_too_large():
    # 50,000 one-row linears: their descriptors alone need more than the
    # static workspace
    M, L = 1, 50000
    packed = torch.zeros(16, dtype=torch.uint8, device=DEV)
    f = torch.zeros(4, dtype=torch.float32, device=DEV)
    i = torch.zeros(4, dtype=torch.int32, device=DEV)
    q = torch.zeros(64, dtype=torch.int8, device=DEV)
    y = torch.zeros(4, dtype=torch.float32, device=DEV)
    d = tern.make_desc(packed, f, i, 1, 64, q, 64, f, i, y, 1)
    with pytest.raises(tern.TernError) as err:
        tern.tern_linear_stack_prepare_static([d] * L, M)
    assert err.value.status == tern.TERN_ERR_RANGE
