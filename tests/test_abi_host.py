"""C ABI checks that need no GPU: the library loads, exports what the header
declares, and argument errors come back as status codes before any launch
(every call below fails validation, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

from packed_bit_gemv_tern_amd import tern

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tern.h")


def header_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tern_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return tern.library()


def test_header_lists_the_four_calls_and_helpers():
    names = header_functions()
    for n in ("tern_pack", "tern_gemv", "tern_gemm_smallM", "tern_linear_stack"):
        assert n in names
    assert set(names) == set(tern.EXPORTS)


def test_header_constants_match_the_binding():
    with open(HEADER) as f:
        defs = dict(re.findall(r"^#define (TERN\w+) (\d+)\s*$", f.read(), flags=re.M))
    assert defs, "no constants found"
    for name, value in defs.items():
        assert getattr(tern, name) == int(value), name


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_row_bytes(lib):
    for K, ld in [(0, 0), (-3, 0), (1, 16), (64, 16), (65, 32), (4096, 1024), (12288, 3072)]:
        assert tern.tern_row_bytes(K) == ld


def test_status_strings(lib):
    for st in range(8):
        assert tern.status_string(st) != "unknown status"

    assert tern.status_string(99) == "unknown status"
    assert lib.tern_last_hip_error() == 0


A16 = 0x10000        # a 16-byte-aligned fake device address (never dereferenced)
ODD = 0x10008        # 8-byte aligned only
S = None             # default stream


def gemm(lib, packed=A16, s_row=A16, rowsum=A16, N=16, K=64, M=2, q=A16, ldq=64, s_act=A16,
         z=A16, y=A16, ldy=16, acc=None, path=0):
    return lib.tern_gemm_smallM(packed, s_row, rowsum, N, K, M, q, ldq, s_act, z, y, ldy, acc,
                                path, S)


def test_gemm_argument_errors(lib):
    assert gemm(lib, K=0) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, K=-5) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, N=-1) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, M=-1) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, K=tern.TERN_MAX_K + 1) == tern.TERN_ERR_RANGE
    assert gemm(lib, N=2 ** 31) == tern.TERN_ERR_RANGE
    for field in ("packed", "s_row", "rowsum", "q", "s_act", "z", "y"):
        assert gemm(lib, **{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert gemm(lib, ldq=63) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, ldy=15) == tern.TERN_ERR_INVALID_ARG
    assert gemm(lib, packed=ODD) == tern.TERN_ERR_ALIGNMENT
    assert gemm(lib, q=ODD) == tern.TERN_ERR_ALIGNMENT
    assert gemm(lib, ldq=72) == tern.TERN_ERR_ALIGNMENT
    assert gemm(lib, y=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert gemm(lib, acc=A16 + 1) == tern.TERN_ERR_ALIGNMENT
    assert gemm(lib, path=tern.TERN_PATH_VALU, M=tern.TERN_VALU_MAX_M + 1) == tern.TERN_ERR_UNSUPPORTED
    assert gemm(lib, path=7) == tern.TERN_ERR_UNSUPPORTED


def test_empty_problems_enqueue_nothing(lib):
    # N == 0 or M == 0 is valid and returns before any launch, even with
    # null buffers
    assert gemm(lib, N=0, packed=None, s_row=None, rowsum=None, y=None) == tern.TERN_OK
    assert gemm(lib, M=0, q=None, s_act=None, z=None, y=None) == tern.TERN_OK
    assert lib.tern_gemv(None, None, None, 0, 64, None, None, None, None, None, S) == tern.TERN_OK
    assert lib.tern_pack(None, 0, 64, 64, None, None, None, S) == tern.TERN_OK
    assert lib.tern_unpack(None, 0, 64, None, 64, S) == tern.TERN_OK


def test_gemv_argument_errors(lib):
    assert lib.tern_gemv(A16, A16, A16, 8, 0, A16, A16, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_gemv(ODD, A16, A16, 8, 64, A16, A16, A16, A16, None, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_gemv(A16, A16, A16, 8, 64, None, A16, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG


def test_pack_unpack_validate_errors(lib):
    assert lib.tern_pack(A16, 4, 64, 63, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_pack(A16, 4, 0, 64, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_pack(A16, 4, 64, 64, ODD, A16, None, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack(A16, 4, 64, 64, A16, A16 + 2, None, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack(A16, 4, 64, 64, A16, A16, A16 + 1, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack(None, 4, 64, 64, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_unpack(A16, 4, 64, A16, 10, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_unpack(ODD, 4, 64, A16, 64, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_validate(A16, 4, 64, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_validate(A16, 4, 64, A16 + 2, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_validate(ODD, 4, 64, A16, S) == tern.TERN_ERR_ALIGNMENT


def _desc(**kw):
    d = tern.tern_linear_desc()
    d.packed = d.s_row = d.rowsum = d.q = d.s_act = d.z = d.y = A16
    d.N, d.K, d.ldq, d.ldy = 16, 64, 64, 16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_stack_prepare_errors(lib):
    plan = tern.tern_stack_plan()
    arr = (tern.tern_linear_desc * 2)(_desc(), _desc(K=0))
    assert lib.tern_linear_stack_prepare(arr, 2, 1, 0, A16, 1 << 20, ctypes.byref(plan), S) \
        == tern.TERN_ERR_INVALID_ARG
    arr = (tern.tern_linear_desc * 2)(_desc(), _desc(packed=ODD))
    assert lib.tern_linear_stack_prepare(arr, 2, 1, 0, A16, 1 << 20, ctypes.byref(plan), S) \
        == tern.TERN_ERR_ALIGNMENT
    arr = (tern.tern_linear_desc * 1)(_desc())
    assert lib.tern_linear_stack_prepare(arr, 1, 1, 0, None, 1 << 20, ctypes.byref(plan), S) \
        == tern.TERN_ERR_WORKSPACE
    assert lib.tern_linear_stack_prepare(arr, 1, 1, 0, A16 + 16, 1 << 20, ctypes.byref(plan), S) \
        == tern.TERN_ERR_WORKSPACE
    assert lib.tern_linear_stack_prepare(arr, 1, 9, tern.TERN_PATH_VALU, A16, 1 << 20,
                                         ctypes.byref(plan), S) == tern.TERN_ERR_UNSUPPORTED
    assert lib.tern_linear_stack_prepare(arr, 1, 1, 0, A16, 1 << 20, None, S) \
        == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_linear_stack(None, S) == tern.TERN_ERR_INVALID_ARG


def test_stack_fused_input_errors(lib):
    # descriptors naming an fp32 input x: checked before anything is launched
    plan = tern.tern_stack_plan()
    X = 0x20000

    def prep(*descs, M=2):
        arr = (tern.tern_linear_desc * len(descs))(*descs)
        return lib.tern_linear_stack_prepare(arr, len(descs), M, 0, A16, 1 << 20, ctypes.byref(plan), S)

    assert prep(_desc(x=X, ldx=63)) == tern.TERN_ERR_INVALID_ARG           # rows shorter than K
    assert prep(_desc(x=X + 2, ldx=64)) == tern.TERN_ERR_ALIGNMENT
    assert prep(_desc(x=X, ldx=2 ** 31)) == tern.TERN_ERR_RANGE
    assert prep(_desc(x=X, ldx=64, ldq=72)) == tern.TERN_ERR_ALIGNMENT     # q rows of 16-byte multiples
    # a linear without rows still has its input written, so its q is checked
    assert prep(_desc(x=X, ldx=64, N=0, q=None)) == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64, N=0, q=A16 + 8)) == tern.TERN_ERR_ALIGNMENT
    # one q buffer, two different inputs or scales
    assert prep(_desc(x=X, ldx=64), _desc(x=X + 1024, ldx=64)) == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64), _desc(x=X, ldx=80)) == tern.TERN_ERR_INVALID_ARG
    # the SwiGLU gate's second input: never without x, 4-byte aligned, one per q buffer
    assert prep(_desc(x_up=X)) == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64, x_up=X + 4096 + 2)) == tern.TERN_ERR_ALIGNMENT
    assert prep(_desc(x=X, ldx=64, x_up=X + 4096), _desc(x=X, ldx=64)) == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64, x_up=X + 4096), _desc(x=X, ldx=64, x_up=X + 8192)) \
        == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64), _desc(s_act=A16 + 64)) == tern.TERN_ERR_INVALID_ARG
    assert prep(_desc(x=X, ldx=64), _desc(K=128, ldq=128)) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_linear_stack_status(None, S) == tern.TERN_ERR_INVALID_ARG


def test_stack_empty_plan(lib):
    plan = tern.tern_stack_plan()
    arr = (tern.tern_linear_desc * 1)(_desc())
    assert lib.tern_linear_stack_prepare(arr, 0, 1, 0, None, 0, ctypes.byref(plan), S) == tern.TERN_OK
    assert plan.L == 0 and plan.workers == 0 and plan.bytes == 0
    assert lib.tern_linear_stack(ctypes.byref(plan), S) == tern.TERN_OK
    assert lib.tern_linear_stack_prepare(arr, 1, 0, 0, None, 0, ctypes.byref(plan), S) == tern.TERN_OK
    assert lib.tern_linear_stack(ctypes.byref(plan), S) == tern.TERN_OK
    assert lib.tern_linear_stack_status(ctypes.byref(plan), S) == tern.TERN_OK


def test_read_probe_argument_errors(lib):
    sink = A16
    assert lib.tern_read_probe(None, 1024, sink, 4, 8, 1, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_read_probe(A16, 1000, sink, 4, 8, 1, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_read_probe(A16, 1024, sink, 0, 8, 1, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_read_probe(A16, 1024, sink, 9, 8, 1, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_read_probe(A16, 1024, sink, 4, 5, 1, S) == tern.TERN_ERR_UNSUPPORTED
    assert lib.tern_read_probe(ODD, 1024, sink, 4, 8, 1, S) == tern.TERN_ERR_ALIGNMENT


def head(lib, W=A16, s_row=A16, rowsum=A16, N=16, K=64, ldw=64, M=2, q=A16, ldq=64, s_act=A16,
         z=A16, y=A16, ldy=16, acc=None):
    return lib.tern_head_gemv(W, s_row, rowsum, N, K, ldw, M, q, ldq, s_act, z, y, ldy, acc, S)


def test_head_argument_errors(lib):
    assert head(lib, N=0) == tern.TERN_OK and head(lib, M=0) == tern.TERN_OK  # empty problems
    assert head(lib, K=0) == tern.TERN_ERR_INVALID_ARG
    assert head(lib, ldw=48) == tern.TERN_ERR_INVALID_ARG
    assert head(lib, M=tern.TERN_HEAD_MAX_M + 1) == tern.TERN_ERR_UNSUPPORTED
    assert head(lib, K=tern.TERN_HEAD_MAX_K + 1, ldw=tern.TERN_HEAD_MAX_K + 16) == tern.TERN_ERR_RANGE
    assert head(lib, ldw=(1 << 28) + 16) == tern.TERN_ERR_RANGE
    for field in ("W", "s_row", "rowsum", "q", "s_act", "z", "y"):
        assert head(lib, **{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert head(lib, ldq=40) == tern.TERN_ERR_INVALID_ARG
    assert head(lib, ldy=8) == tern.TERN_ERR_INVALID_ARG
    assert head(lib, W=ODD) == tern.TERN_ERR_ALIGNMENT
    assert head(lib, ldw=72) == tern.TERN_ERR_ALIGNMENT
    assert head(lib, ldq=72) == tern.TERN_ERR_ALIGNMENT
    assert head(lib, acc=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_head_rowsum(A16, 4, 64, 32, A16, S) == tern.TERN_ERR_INVALID_ARG   # ldw < K
    assert lib.tern_head_rowsum(None, 4, 64, 64, A16, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_head_rowsum(A16, 0, 64, 64, None, S) == tern.TERN_OK


def test_blocked_argument_errors(lib):
    def blk(packed=A16, s_b=A16, rb=A16, N=4, K=256, B=128, q=A16, s_act=A16, z=A16, y=A16):
        return lib.tern_gemv_blocked(packed, s_b, rb, N, K, B, q, s_act, z, y, S)
    assert blk(N=0) == tern.TERN_OK
    for B in (0, 32, 96, 192, 8192):
        assert blk(B=B) == tern.TERN_ERR_INVALID_ARG, B
    assert blk(K=tern.TERN_BLOCK_MAX_K + 1) == tern.TERN_ERR_RANGE
    for field in ("packed", "s_b", "rb", "q", "s_act", "z", "y"):
        assert blk(**{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert blk(packed=ODD) == tern.TERN_ERR_ALIGNMENT
    assert blk(q=ODD) == tern.TERN_ERR_ALIGNMENT
    assert blk(s_b=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_block_rowsum(A16, 4, 256, 100, A16, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_block_rowsum(A16, 4, tern.TERN_BLOCK_MAX_K + 1, 128, A16, S) == tern.TERN_ERR_RANGE


def test_quantize_argument_errors(lib):
    def qa(x=A16, M=2, K=64, ldx=64, q=A16, ldq=64, s=A16, z=A16):
        return lib.tern_quantize_act(x, M, K, ldx, q, ldq, s, z, S)
    assert qa(M=0) == tern.TERN_OK
    assert qa(K=0) == tern.TERN_ERR_INVALID_ARG
    assert qa(ldx=63) == tern.TERN_ERR_INVALID_ARG
    assert qa(ldq=63) == tern.TERN_ERR_INVALID_ARG
    for field in ("x", "q", "s", "z"):
        assert qa(**{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert qa(x=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert qa(s=A16 + 1) == tern.TERN_ERR_ALIGNMENT


def test_packed5_row_bytes_and_argument_errors(lib):
    for K, ld in [(0, 0), (-1, 0), (1, 16), (80, 16), (81, 32), (4096, 832), (12288, 2464)]:
        assert tern.tern_row_bytes5(K) == ld, K
    assert lib.tern_pack5(A16, 4, 64, 63, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_pack5(A16, 4, 0, 64, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    K5 = tern.TERN5_MAX_K + 1
    assert lib.tern_pack5(A16, 4, K5, K5, A16, A16, None, S) == tern.TERN_ERR_RANGE
    assert lib.tern_pack5(A16, 4, 64, 64, ODD, A16, None, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack5(A16, 4, 64, 64, A16, A16 + 2, None, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack5(A16, 4, 64, 64, A16, A16, A16 + 1, S) == tern.TERN_ERR_ALIGNMENT
    assert lib.tern_pack5(None, 4, 64, 64, A16, A16, None, S) == tern.TERN_ERR_INVALID_ARG
    assert lib.tern_pack5(None, 0, 64, 64, None, None, None, S) == tern.TERN_OK

    def g5(packed=A16, s_row=A16, rs=A16, N=8, K=100, q=A16, s_act=A16, z=A16, y=A16, acc=None):
        return lib.tern_gemv5(packed, s_row, rs, N, K, q, s_act, z, y, acc, S)
    assert g5(N=0) == tern.TERN_OK
    assert g5(K=0) == tern.TERN_ERR_INVALID_ARG
    assert g5(N=-1) == tern.TERN_ERR_INVALID_ARG
    assert g5(K=tern.TERN5_MAX_K + 1) == tern.TERN_ERR_RANGE
    for field in ("packed", "s_row", "rs", "q", "s_act", "z", "y"):
        assert g5(**{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert g5(packed=ODD) == tern.TERN_ERR_ALIGNMENT
    assert g5(q=ODD) == tern.TERN_ERR_ALIGNMENT
    assert g5(y=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert g5(acc=A16 + 1) == tern.TERN_ERR_ALIGNMENT


def test_weight_quantiser_argument_errors(lib):
    def wq(W=A16, N=4, K=64, ldw=64, B=16, w=A16, ldt=64, s=A16):
        return lib.tern_quantize_weights(W, N, K, ldw, B, w, ldt, s, S)
    assert wq(N=0) == tern.TERN_OK
    assert wq(K=0) == tern.TERN_ERR_INVALID_ARG
    assert wq(B=0) == tern.TERN_ERR_INVALID_ARG
    assert wq(ldw=63) == tern.TERN_ERR_INVALID_ARG
    assert wq(ldt=63) == tern.TERN_ERR_INVALID_ARG
    for field in ("W", "w", "s"):
        assert wq(**{field: None}) == tern.TERN_ERR_INVALID_ARG, field
    assert wq(W=A16 + 2) == tern.TERN_ERR_ALIGNMENT
    assert wq(s=A16 + 1) == tern.TERN_ERR_ALIGNMENT
    # one thread per (row, block) in one launch, which counts at most
    # 2^32 - 1 work-items: 2^24 rows x 256 one-column blocks is one too many
    assert wq(N=2 ** 24, K=256, ldw=256, ldt=256, B=1) == tern.TERN_ERR_RANGE
    assert wq(N=2 ** 31 - 1, K=2 ** 20, ldw=2 ** 20, ldt=2 ** 20, B=1) == tern.TERN_ERR_RANGE


def test_dispatch_size_limits(lib):
    # Each launch below would need 2^32 or more work-items (its grid times
    # its 256-thread workgroups): refused up front with TERN_ERR_RANGE.
    n = tern.TERN_MAX_ROWS_PACK + 1  # one wave per row, four rows per workgroup
    assert (n + 3) // 4 * 256 > 2 ** 32 - 1 >= (n - 1 + 3) // 4 * 256
    assert lib.tern_pack(A16, n, 64, 64, A16, A16, None, S) == tern.TERN_ERR_RANGE
    assert lib.tern_unpack(A16, n, 64, A16, 64, S) == tern.TERN_ERR_RANGE
    assert lib.tern_validate(A16, n, 64, A16, S) == tern.TERN_ERR_RANGE
    assert lib.tern_head_rowsum(A16, 2 ** 26 - 3, 64, 64, A16, S) == tern.TERN_ERR_RANGE
    assert lib.tern_pack5(A16, 2 ** 26 - 3, 64, 64, A16, A16, None, S) == tern.TERN_ERR_RANGE
    # 1.6-bit GEMV at K = 100: 16 rows per wave, four waves per workgroup
    assert lib.tern_gemv5(A16, A16, A16, 2 ** 30, 100, A16, A16, A16, A16, None, S) == tern.TERN_ERR_RANGE
    # block row sums: one thread per (row, block)
    assert lib.tern_block_rowsum(A16, 2 ** 26, 4096, 64, A16, S) == tern.TERN_ERR_RANGE
    # activation quantiser: one workgroup per token
    assert lib.tern_quantize_act(A16, 2 ** 24, 64, 64, A16, 64, A16, A16, S) == tern.TERN_ERR_RANGE
