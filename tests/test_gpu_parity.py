"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Integer results (packed bytes, row sums, int32 accumulators, counts) must be
bit-exact; fp32 outputs must lie within 1e-6 relative of the oracle's fp64
value and match its ordered fp32 evaluation bit for bit.
"""
import numpy as np
import pytest

import oracle
from packed_bit_gemv_tern_amd import synth, tern

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import (DEV, Uploaded, assert_parity, gpu_pack, oracle_ref,  # noqa: E402
                      to_dev)
from test_oracle_pins import read_packed_rows  # noqa: E402


def make(N, K, M, seed=0, p0=0.626):
    return synth.make_linear(seed, N, K, N, K, p0, M, "t%dx%dx%d" % (N, K, M))


# ------------------------------------------------------------------ pack --

def test_pack_golden_rows():
    for K, w, hx, rs in read_packed_rows():
        packed, rowsum, bad = gpu_pack(w[None, :])
        torch.cuda.synchronize()
        assert packed.cpu().numpy().tobytes().hex() == hx, K
        assert int(rowsum.item()) == rs and int(bad.item()) == 0


@pytest.mark.parametrize("K", list(range(1, 131)) + [512, 1024, 2048, 3072, 4096, 12288])
def test_pack_matches_oracle(K):
    rng = np.random.default_rng(K)
    N = 37
    w = synth.ternary(rng, N, K, 0.626)
    packed, rowsum, bad = gpu_pack(w)
    rp, rr, rb = oracle.pack(w)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(rowsum.cpu().numpy(), rr)
    assert int(bad.item()) == rb == 0


def test_pack_strided_unaligned_rows_and_bad_values():
    rng = np.random.default_rng(3)
    N, K, ldw = 9, 77, 83  # rows neither 16-byte aligned nor a 16 multiple long
    full = rng.integers(-1, 2, (N, ldw)).astype(np.int8)
    full[2, 5] = 7
    full[4, 76] = -128
    full[6, 80] = 99  # past K: ignored
    wd = to_dev(full)
    packed = torch.empty((N, tern.tern_row_bytes(K)), dtype=torch.uint8, device=DEV)
    rowsum = torch.empty(N, dtype=torch.int32, device=DEV)
    bad = torch.empty(1, dtype=torch.int32, device=DEV)
    tern.tern_pack(wd, N, K, ldw, packed, rowsum, bad)
    rp, rr, rb = oracle.pack(full[:, :K])
    torch.cuda.synchronize()
    assert rb == 2 and int(bad.item()) == 2
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(rowsum.cpu().numpy(), rr)


def test_unpack_roundtrip_and_validate():
    rng = np.random.default_rng(4)
    for K in (1, 15, 64, 100, 4096):
        N = 21
        w = synth.ternary(rng, N, K, 0.626)
        packed, _, _ = gpu_pack(w)
        back = torch.zeros((N, K + 3), dtype=torch.int8, device=DEV)
        tern.tern_unpack(packed, N, K, back, K + 3)
        counts = torch.full((2,), -1, dtype=torch.int32, device=DEV)
        tern.tern_validate(packed, N, K, counts)
        torch.cuda.synchronize()
        assert np.array_equal(back.cpu().numpy()[:, :K], w)
        assert counts.cpu().tolist() == [0, 0]
        # corrupt: one 11 code in a real column, two non-01 padding fields
        bad = packed.cpu().numpy().copy()
        bad[3, 0] |= 0x03
        extra_pad = 0
        if K % 64:
            j = K  # first padding column: byte 4*(j//16) + j%4, shift 2*((j%16)//4)
            bad[5, 4 * (j // 16) + j % 4] &= ~(3 << (2 * ((j % 16) // 4))) & 0xFF
            extra_pad = 1
        badd = to_dev(bad)
        tern.tern_validate(badd, N, K, counts)
        torch.cuda.synchronize()
        assert counts.cpu().tolist() == list(oracle.validate(bad, N, K)) == [1, extra_pad]
        tern.tern_unpack(badd, N, K, back, K + 3)
        ref, inv = oracle.unpack(bad, N, K)
        torch.cuda.synchronize()
        assert inv == 1 and np.array_equal(back.cpu().numpy()[:, :K], ref)


# ------------------------------------------------------------------ gemv --

def test_single_gemv_256x512_seed0():
    lin = synth.single_gemv_case()
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "256x512")


GEMV_K = [1, 7, 63, 64, 65, 100, 500, 512, 1000, 1024, 1500, 2048, 2100, 3072, 3100, 4096,
          4200, 8192, 12288, 16384, 16400, 20000]


@pytest.mark.parametrize("K", GEMV_K)
@pytest.mark.parametrize("N", [1, 5, 37, 300])
def test_gemv_shapes(N, K):
    lin = make(N, K, 1, seed=K * 7 + N)
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "gemv N=%d K=%d" % (N, K))


def test_gemv_extreme_values():
    # worst-case magnitudes: q at -128 / 127, |z| = 255, all-nonzero rows
    for qv, zv in [(-128, 255), (127, -255), (-128, -255)]:
        N, K = 64, 12288
        w = np.where(np.arange(K)[None, :] % 2 == 0, 1, -1).astype(np.int8).repeat(N, 0)
        w[1] = 1
        w[2] = -1
        w[3] = 0
        lin = synth.Linear("x", w, np.full(N, 0.1, np.float32), np.full((1, K), qv, np.int8),
                           np.array([0.03], np.float32), np.array([zv], np.int32))
        up = Uploaded(lin)
        up.run()
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "extreme q=%d z=%d" % (qv, zv))


def test_gemv_zero_weights_give_positive_zero():
    N, K = 40, 4096
    lin = synth.Linear("zero", np.zeros((N, K), np.int8), np.full(N, 0.05, np.float32),
                       np.full((1, K), 9, np.int8), np.array([0.02], np.float32),
                       np.array([3], np.int32))
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    assert not acc.any()
    assert np.all(y.view(np.uint32) == 0)


def test_gemv_acc_optional_and_repeatable():
    lin = make(300, 4096, 1, seed=11)
    up = Uploaded(lin)
    tern.tern_gemv(up.packed, up.s_row, up.rowsum, lin.N, lin.K, up.q, up.s_act, up.z, up.y, None)
    torch.cuda.synchronize()
    y1 = up.y.cpu().numpy().copy()
    up.run()
    y2, acc = up.results()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert_parity(y2, acc, oracle_ref(lin), "repeat")


# --------------------------------------------------------------- small M --

SMALLM_K = [64, 100, 576, 1024, 3072, 4096, 4160, 12288]


@pytest.mark.parametrize("M", list(range(1, 17)) + [17, 31, 64])
@pytest.mark.parametrize("K", SMALLM_K)
def test_gemm_mfma(M, K):
    N = 70
    lin = make(N, K, M, seed=M * 31 + K)
    up = Uploaded(lin, ldy_extra=5)
    up.run(tern.TERN_PATH_MFMA)
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "mfma M=%d K=%d" % (M, K))
    # columns past N of each output row are untouched
    torch.cuda.synchronize()
    assert torch.isnan(up.y[:, N:]).all() and (up.acc[:, N:] == -7).all()


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("K", [64, 100, 4096, 12288, 20000])
def test_gemm_valu(M, K):
    N = 45
    lin = make(N, K, M, seed=M * 13 + K)
    up = Uploaded(lin, ldy_extra=3)
    up.run(tern.TERN_PATH_VALU)
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "valu M=%d K=%d" % (M, K))


@pytest.mark.parametrize("M", [64, 512])
def test_gemm_prefill(M):
    N, K = 200, 4096
    lin = make(N, K, M, seed=M)
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "prefill M=%d" % M)


def test_gemm_prefill_512_row_tiles():
    # a single call with enough 512 x 128 tiles (96 x 8 = 768, three per CU)
    # for the 512-row tile, ragged in M
    N, K, M = 49152, 64, 1000
    lin = make(N, K, M, seed=11)
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    assert_parity(y, acc, oracle_ref(lin), "prefill N=%d M=%d" % (N, M))


def test_gemm_empty_problems():
    y = torch.full((4, 8), 5.0, device=DEV)
    dummy8 = torch.zeros(64, dtype=torch.int8, device=DEV)
    dummyf = torch.zeros(8, dtype=torch.float32, device=DEV)
    dummyi = torch.zeros(8, dtype=torch.int32, device=DEV)
    packed = torch.zeros(16 * 8, dtype=torch.uint8, device=DEV)
    tern.tern_gemm_smallM(packed, dummyf, dummyi, 0, 64, 4, dummy8, 64, dummyf, dummyi, y, 8)
    tern.tern_gemm_smallM(packed, dummyf, dummyi, 8, 64, 0, dummy8, 64, dummyf, dummyi, y, 8)
    torch.cuda.synchronize()
    assert (y == 5.0).all()


# ----------------------------------------------------------------- stack --

def _stack_case(model, layers, M, seed=0):
    lins = synth.make_stack(seed, M, model=model, layers=layers, threads=8)
    ups = [Uploaded(lin) for lin in lins]
    return lins, ups


@pytest.mark.parametrize("path", [tern.TERN_PATH_AUTO, tern.TERN_PATH_VALU, tern.TERN_PATH_MFMA])
@pytest.mark.parametrize("M", [1, 8])
def test_stack_06b_two_layers(M, path):
    lins, ups = _stack_case("0.6b", 2, M)
    L = len(ups)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(L, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws, path)
    assert plan.L == L and plan.workers > 0
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "stack %s M=%d" % (lin.name, M))


@pytest.mark.parametrize("M", [1, 8, 12, 16])
def test_stack_8b_one_layer(M):
    lins, ups = _stack_case("8b", 1, M, seed=5)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8,
                     device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    # one layer at M = 8 is small enough that the K = 12,288 down projection
    # is split per window (partial sums through the output buffer); at 12
    # and 16 tokens the layer takes the 16-token window kernel, which never
    # splits
    assert plan.kernel == (16 + 11 if M > 8 else plan.kernel)
    assert plan.splits == (1 if M == 8 else 0)
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)  # a second launch over the same plan
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "8b layer %s M=%d" % (lin.name, M))


@pytest.mark.parametrize("M", [2, 5, 8, 17, 64, 130])
def test_stack_split_windows(M):
    # two K = 12,288 linears and a K = 8,192 one among short ones: split, and
    # launched twice (the fill kernel must clear the previous sums)
    specs = [(300, 12288, 1), (64, 4096, 2), (257, 8192, 3), (40, 12288, 4), (100, 1024, 5)]
    lins = [synth.make_linear(13, s, 0, N, K, 0.626, M, "s%d" % s) for (N, K, s) in specs]
    ups = [Uploaded(lin) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws, tern.TERN_PATH_MFMA)
    assert plan.splits == 3
    for _ in range(3):
        tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "split %s M=%d" % (lin.name, M))


@pytest.mark.parametrize("M", [20, 100])
def test_stack_split_ragged_k_prefill(M):
    # prefill GEMM: K = 8,384 in windows of 4,096, 4,096 and 192 columns; a
    # ragged K (not split) and a short one beside it
    specs = [(200, 8384, 1), (70, 4100, 2), (33, 100, 3), (90, 12288, 4)]
    lins = [synth.make_linear(17, s, 0, N, K, 0.626, M, "r%d" % s) for (N, K, s) in specs]
    ups = [Uploaded(lin) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws, tern.TERN_PATH_MFMA)
    assert plan.splits == 2
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "split %s M=%d" % (lin.name, M))


# Stacks whose linears return y only: the activation-window kernel (M <= 8)
# holds such outputs in registers until a worker's run ends (every other
# stack test also asks for acc, which is stored at once).

@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_stack_y_only(M):
    lins = synth.make_stack(4, M, model="0.6b", layers=2, threads=8)
    ups = [Uploaded(lin, ldy_extra=3, with_acc=False) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert acc is None
        assert_parity(y, None, oracle_ref(lin), "y-only %s M=%d" % (lin.name, M))
        assert torch.isnan(up.y[:, lin.N:]).all()  # nothing past N written


@pytest.mark.parametrize("M", [4, 8])
def test_stack_y_only_8b_layer_and_mixed_acc(M):
    # one 8B layer (its down projection is split: partial sums stored at
    # once beside held outputs); every other linear also asks for acc
    lins, _ = _stack_case("8b", 1, M, seed=6)
    ups = [Uploaded(lin, ldy_extra=1, with_acc=(i % 2 == 1)) for i, lin in enumerate(lins)]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    assert plan.splits == 1
    for _ in range(2):
        tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "8b mixed %s M=%d" % (lin.name, M))
        assert torch.isnan(up.y[:, lin.N:]).all()


def test_stack_y_only_more_rows_than_held():
    # K = 64 rows are cheap, so each worker takes far more 256-row units than
    # the 24 a wave holds: the held outputs are stored when the buffer fills
    # as well as at the end of the run
    M = 8
    specs = [(1200007, 64, 1), (1199993, 64, 2), (300, 4096, 3)]
    lins = [synth.make_linear(21, s, 0, N, K, 0.626, M, "o%d" % s) for (N, K, s) in specs]
    ups = [Uploaded(lin, with_acc=False) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    units = sum(-(-N // 256) for (N, _, _) in specs)
    assert units > 24 * plan.workers * 1.2, (units, plan.workers)
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, _ = up.results()
        assert_parity(y, None, oracle_ref(lin), "overflow %s" % lin.name)


@pytest.mark.parametrize("M", [9, 12, 16])
@pytest.mark.parametrize("with_acc", [True, False])
def test_stack_16_token_window(M, with_acc):
    # six 0.6B layers at 9..16 tokens: the window kernel with all 16
    # activation rows staged, one workgroup per CU; launched twice
    lins = synth.make_stack(8, M, model="0.6b", layers=6, threads=8)
    ups = [Uploaded(lin, ldy_extra=3, with_acc=with_acc) for lin in lins]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert plan.splits == 0 and plan.grid == cus // 8 * 8, (plan.grid, cus)
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "16-token %s M=%d" % (lin.name, M))
        assert torch.isnan(up.y[:, lin.N:]).all()


def test_stack_mixed_shapes_and_empty_linear():
    specs = [(5, 1, 1), (300, 4096, 2), (0, 64, 3), (77, 100, 4), (40, 12288, 5), (129, 1000, 6)]
    for M in (1, 3, 8, 12, 40, 130):
        lins = [synth.make_linear(9, s, 0, N, K, 0.626, M, "m%d" % s) for (N, K, s) in specs]
        ups = [Uploaded(lin) for lin in lins if lin.N > 0]
        lins = [lin for lin in lins if lin.N > 0]
        ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups) + 1, M),
                         dtype=torch.uint8, device=DEV)
        descs = [u.desc() for u in ups]
        empty = tern.make_desc(ups[0].packed, ups[0].s_row, ups[0].rowsum, 0, 64, ups[0].q,
                               ups[0].ldq, ups[0].s_act, ups[0].z, ups[0].y, ups[0].ldy)
        plan = tern.tern_linear_stack_prepare(descs[:2] + [empty] + descs[2:], M, ws)
        tern.tern_linear_stack(plan)
        for lin, up in zip(lins, ups):
            y, acc = up.results()
            assert_parity(y, acc, oracle_ref(lin), "mixed %s M=%d" % (lin.name, M))


# Linears of a layer that read one input (q/k/v, gate/up) given one
# activation buffer: the window kernel stages it once for consecutive
# segments of a workgroup that read it.  0.6B shapes: every window ends past K
# (K = 1,024, 2,048, 3,072), so the staged tail beyond K must read as zero.

@pytest.mark.parametrize("M", [2, 5, 8])
def test_stack_shared_inputs_06b(M):
    from packed_bit_gemv_tern_amd.stack import DeviceStack
    st = DeviceStack("0.6b", layers=3, seed=7, threads=8)
    b = st.bind(M, with_acc=False, share_inputs=True)
    b_ind = st.bind(M, with_acc=False)
    assert b.plan.restages <= b_ind.plan.restages  # (a shallow stack gives each workgroup ~1 segment)
    b.run()
    b.run()
    torch.cuda.synchronize()
    for i, (layer, idx, name, N, K, p0) in enumerate(st.specs):
        w, s_row = synth.make_weights(7, layer, idx, N, K, p0)
        q, s_act, z = synth.make_activations(7, layer, synth.INPUT_LEADER[idx], K, M)
        packed, rowsum, _ = oracle.pack(w)
        ref = oracle.linear(packed, s_row, rowsum, K, q, s_act, z)
        assert_parity(b.y[i].cpu().numpy(), None, ref, "shared %d.%s M=%d" % (layer, name, M))


# Window-major order: linears of several whole 4,096-column windows whose
# outputs are held (y only) are walked by each workgroup a window at a time
# over a group of its units, the int32 sums of the earlier windows waiting in
# the held slots.  About three such units per workgroup here, with 2, 3 and 4
# windows; the linear that also returns acc walks unit by unit.

@pytest.mark.timeout(300)
@pytest.mark.parametrize("M", [2, 5, 8])
def test_stack_window_major(M):
    specs = [(98304, 8192, 1), (40960, 12288, 2), (16384, 16384, 3), (700, 12288, 4)]
    lins = [synth.make_linear(31, sd, 0, N, K, 0.626, M, "wm%d" % sd) for (N, K, sd) in specs]
    ups = [Uploaded(lin, with_acc=(i == 3)) for i, lin in enumerate(lins)]
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(len(ups), M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([u.desc() for u in ups], M, ws)
    assert plan.splits == 0
    # window-major: fewer window loads than units x windows
    unit_windows = sum((N + 255) // 256 * (K // 4096) for (N, K, _) in specs)
    assert plan.restages < unit_windows // 2
    tern.tern_linear_stack(plan)
    tern.tern_linear_stack(plan)
    for lin, up in zip(lins, ups):
        y, acc = up.results()
        assert_parity(y, acc, oracle_ref(lin), "window-major %s M=%d" % (lin.name, M))


# Long K on every path: past 2^21 columns a plane-scaled int32 sum of a whole
# row (16 * sum(c*q) for code plane 2 on the M <= 8 window kernel) would pass
# 2^31, while the exact result is well inside int32.  All +1 weights with
# q = -128 reach that bound; |acc| > 2^24 here, so the conversion to float
# rounds (to nearest even on both sides) and y is compared bit for bit.

LONG_K = 2_101_248  # 513 activation windows of 4,096 columns


def _long_k_linear(M):
    N, K = 16, LONG_K
    w = np.ones((N, K), np.int8)
    w[1] = -1
    w[2, 1::2] = 0
    w[3] = np.where(np.arange(K) % 3 == 0, -1, 1)
    w[4:] = synth.ternary(np.random.default_rng(77), N - 4, K, 0.626)
    q = np.full((M, K), -128, np.int8)
    if M > 1:
        q[1] = 127
    z = np.array([0, 255, -3, 5, 0, 1, 2, 3][:M], np.int32)
    return synth.Linear("longK", w, np.full(N, 0.01, np.float32), q,
                        np.full(M, 0.02, np.float32), z)


def _long_k_check(y, acc, lin, ctx):
    packed, rowsum, _ = oracle.pack(lin.w)
    racc, ry32, _ = oracle.linear(packed, lin.s_row, rowsum, lin.K, lin.q, lin.s_act, lin.z,
                                  check=False)
    assert abs(int(racc[0, 0])) > 2 ** 24  # the case the test is for
    if acc is not None:
        bad = np.argwhere(acc != racc)
        assert bad.size == 0, "%s acc mismatch at %s: gpu %s oracle %s" % (
            ctx, bad[:5].tolist(), acc[tuple(bad[0])], racc[tuple(bad[0])])
    assert np.array_equal(y.view(np.uint32), ry32.view(np.uint32)), "%s y differs" % ctx


@pytest.mark.parametrize("M", [1, 2, 8])
def test_long_k_past_2_21_columns(M):
    lin = _long_k_linear(M)
    up = Uploaded(lin)
    up.run()
    y, acc = up.results()
    _long_k_check(y, acc, lin, "long K call M=%d" % M)
    # the stack launch, y only (held outputs on the window kernel)
    up2 = Uploaded(lin, with_acc=False)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([up2.desc()], M, ws)
    tern.tern_linear_stack(plan)
    y2, _ = up2.results()
    _long_k_check(y2, None, lin, "long K stack M=%d" % M)


@pytest.mark.parametrize("ldy", [(1 << 29) - 64, 1 << 29])
def test_outputs_near_32bit_offsets(ldy):
    """M = 2 outputs rows ldy apart: (M * ldy * 4) just below 2^32 keeps the
    activation-window kernel (32-bit output offsets); 2^32 sends the call to
    the other MFMA kernel.  Both through gemm_smallM and through the stack."""
    N, K, M = 300, 4096, 2
    lin = make(N, K, M, seed=41)
    up = Uploaded(lin)
    ref = oracle_ref(lin)
    y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((M, ldy), -7, dtype=torch.int32, device=DEV)

    def fetch():
        torch.cuda.synchronize()
        return y[:, :N].cpu().numpy(), acc[:, :N].cpu().numpy()

    tern.tern_gemm_smallM(up.packed, up.s_row, up.rowsum, N, K, M, up.q, up.ldq, up.s_act, up.z,
                          y, ldy, acc, tern.TERN_PATH_MFMA)
    assert_parity(*fetch(), ref, "gemm ldy=%d" % ldy)
    torch.cuda.synchronize()
    assert torch.isnan(y[:, N:N + 64]).all() and torch.isnan(y[:, -64:]).all()

    y.fill_(float("nan"))
    acc.fill_(-7)
    desc = tern.make_desc(up.packed, up.s_row, up.rowsum, N, K, up.q, up.ldq, up.s_act, up.z, y,
                          ldy, acc)
    ws = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=DEV)
    plan = tern.tern_linear_stack_prepare([desc], M, ws, tern.TERN_PATH_MFMA)
    tern.tern_linear_stack(plan)
    assert_parity(*fetch(), ref, "stack ldy=%d" % ldy)
