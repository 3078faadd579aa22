"""ctypes binding of libtern.so (include/tern.h), with the same names.

Argument marshalling only: every step of the computation runs in the HIP
kernels.  torch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  Loading fails loudly when the
shared library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtern.so")

TERN_OK = 0
TERN_ERR_INVALID_ARG = 1
TERN_ERR_ALIGNMENT = 2
TERN_ERR_RANGE = 3
TERN_ERR_UNSUPPORTED = 4
TERN_ERR_WORKSPACE = 5
TERN_ERR_HIP = 6
TERN_ERR_TIMEOUT = 7
TERN_PATH_AUTO, TERN_PATH_VALU, TERN_PATH_MFMA = 0, 1, 2
TERN_MAX_K = 5600000
TERN_VALU_MAX_M = 8
TERN_MAX_ROWS_PACK = 67108860
TERN_STATIC_WORKSPACE_BYTES = 4194304
TERN_BLOCK_MAX_K = 16384
TERN_HEAD_MAX_M = 8
TERN_HEAD_MAX_K = 43803
TERN5_MAX_K = 65520

# Every function include/tern.h declares.
EXPORTS = (
    "tern_row_bytes", "tern_pack", "tern_unpack", "tern_validate", "tern_gemv",
    "tern_gemm_smallM", "tern_linear_stack_workspace_bytes", "tern_linear_stack_prepare",
    "tern_linear_stack", "tern_linear_stack_status", "tern_linear_stack_prepare_static", "tern_block_rowsum", "tern_gemv_blocked", "tern_quantize_act",
    "tern_quantize_weights", "tern_head_rowsum", "tern_head_gemv", "tern_row_bytes5", "tern_pack5", "tern_gemv5",
    "tern_read_probe",
    "tern_status_string", "tern_last_hip_error",
)


class TernError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s (status %d)" % (where, status_string(status), status)
        if status == TERN_ERR_HIP:
            msg += ", hipError %d" % _lib().tern_last_hip_error()
        super().__init__(msg)


class tern_linear_desc(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p), ("s_row", ctypes.c_void_p), ("rowsum", ctypes.c_void_p),
        ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("ldq", ctypes.c_int64),
        ("s_act", ctypes.c_void_p), ("z", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("acc", ctypes.c_void_p),
        ("block", ctypes.c_int64), ("s_block", ctypes.c_void_p), ("rowsum_block", ctypes.c_void_p),
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("x_up", ctypes.c_void_p),
    ]


class tern_stack_plan(ctypes.Structure):
    _fields_ = [
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("L", ctypes.c_int32), ("M", ctypes.c_int32), ("path", ctypes.c_int32),
        ("grid", ctypes.c_int32), ("block", ctypes.c_int32), ("workers", ctypes.c_int32),
        ("segments", ctypes.c_int32), ("kernel", ctypes.c_int32), ("bytes", ctypes.c_int64),
        ("splits", ctypes.c_int32), ("restages", ctypes.c_int32),
    ]


_lock = threading.Lock()
_handle = None


def _lib():
    global _handle
    if _handle is None:
        with _lock:
            if _handle is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        "libtern.so is not built (%s); run `python -m "
                        "packed_bit_gemv_tern_amd.build` first" % LIB_PATH)
                _handle = _declare(ctypes.CDLL(LIB_PATH))
    return _handle


def _declare(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "tern_row_bytes": (i64, [i64]),
        "tern_pack": (i32, [vp, i64, i64, i64, vp, vp, vp, vp]),
        "tern_unpack": (i32, [vp, i64, i64, vp, i64, vp]),
        "tern_validate": (i32, [vp, i64, i64, vp, vp]),
        "tern_gemv": (i32, [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]),
        "tern_gemm_smallM": (i32, [vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp,
                                   i32, vp]),
        "tern_linear_stack_workspace_bytes": (i64, [i64, i64]),
        "tern_linear_stack_prepare": (i32, [ctypes.POINTER(tern_linear_desc), i64, i64, i32,
                                            vp, i64, ctypes.POINTER(tern_stack_plan), vp]),
        "tern_linear_stack": (i32, [ctypes.POINTER(tern_stack_plan), vp]),
        "tern_linear_stack_status": (i32, [ctypes.POINTER(tern_stack_plan), vp]),
        "tern_linear_stack_prepare_static": (i32, [ctypes.POINTER(tern_linear_desc), i64, i64, i32,
                                                   ctypes.POINTER(tern_stack_plan), vp]),
        "tern_block_rowsum": (i32, [vp, i64, i64, i64, vp, vp]),
        "tern_gemv_blocked": (i32, [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp]),
        "tern_quantize_act": (i32, [vp, i64, i64, i64, vp, i64, vp, vp, vp]),
        "tern_quantize_weights": (i32, [vp, i64, i64, i64, i64, vp, i64, vp, vp]),
        "tern_head_rowsum": (i32, [vp, i64, i64, i64, vp, vp]),
        "tern_head_gemv": (i32, [vp, vp, vp, i64, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, vp]),
        "tern_row_bytes5": (i64, [i64]),
        "tern_pack5": (i32, [vp, i64, i64, i64, vp, vp, vp, vp]),
        "tern_gemv5": (i32, [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]),
        "tern_read_probe": (i32, [vp, i64, vp, i32, i32, i32, vp]),
        "tern_status_string": (ctypes.c_char_p, [i32]),
        "tern_last_hip_error": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def status_string(status: int) -> str:
    return _lib().tern_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != TERN_OK:
        raise TernError(status, where)


def _ptr(t):
    """Device address of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


# ------------------------------------------------------------ entry points --

def tern_row_bytes(K: int) -> int:
    return int(_lib().tern_row_bytes(int(K)))


def tern_pack(w, N, K, ldw, packed, rowsum, bad_count=None, stream=None):
    _check(_lib().tern_pack(_ptr(w), N, K, ldw, _ptr(packed), _ptr(rowsum), _ptr(bad_count),
                            _stream(stream)), "tern_pack")


def tern_unpack(packed, N, K, w, ldw, stream=None):
    _check(_lib().tern_unpack(_ptr(packed), N, K, _ptr(w), ldw, _stream(stream)), "tern_unpack")


def tern_validate(packed, N, K, counts, stream=None):
    _check(_lib().tern_validate(_ptr(packed), N, K, _ptr(counts), _stream(stream)),
           "tern_validate")


def tern_gemv(packed, s_row, rowsum, N, K, q, s_act, z, y, acc=None, stream=None):
    _check(_lib().tern_gemv(_ptr(packed), _ptr(s_row), _ptr(rowsum), N, K, _ptr(q), _ptr(s_act),
                            _ptr(z), _ptr(y), _ptr(acc), _stream(stream)), "tern_gemv")


def tern_gemm_smallM(packed, s_row, rowsum, N, K, M, q, ldq, s_act, z, y, ldy, acc=None,
                     path=TERN_PATH_AUTO, stream=None):
    _check(_lib().tern_gemm_smallM(_ptr(packed), _ptr(s_row), _ptr(rowsum), N, K, M, _ptr(q), ldq,
                                   _ptr(s_act), _ptr(z), _ptr(y), ldy, _ptr(acc), int(path),
                                   _stream(stream)), "tern_gemm_smallM")


def tern_block_rowsum(packed, N, K, B, rowsum_b, stream=None):
    _check(_lib().tern_block_rowsum(_ptr(packed), N, K, B, _ptr(rowsum_b), _stream(stream)),
           "tern_block_rowsum")


def tern_gemv_blocked(packed, s_b, rowsum_b, N, K, B, q, s_act, z, y, stream=None):
    _check(_lib().tern_gemv_blocked(_ptr(packed), _ptr(s_b), _ptr(rowsum_b), N, K, B, _ptr(q),
                                    _ptr(s_act), _ptr(z), _ptr(y), _stream(stream)), "tern_gemv_blocked")


def tern_quantize_act(x, M, K, ldx, q, ldq, s_act, z, stream=None):
    _check(_lib().tern_quantize_act(_ptr(x), M, K, ldx, _ptr(q), ldq, _ptr(s_act), _ptr(z),
                                    _stream(stream)), "tern_quantize_act")


def tern_quantize_weights(W, N, K, ldw, B, w, ldt, s_b, stream=None):
    _check(_lib().tern_quantize_weights(_ptr(W), N, K, ldw, B, _ptr(w), ldt, _ptr(s_b), _stream(stream)),
           "tern_quantize_weights")


def tern_head_rowsum(W, N, K, ldw, rowsum, stream=None):
    _check(_lib().tern_head_rowsum(_ptr(W), N, K, ldw, _ptr(rowsum), _stream(stream)),
           "tern_head_rowsum")


def tern_head_gemv(W, s_row, rowsum, N, K, ldw, M, q, ldq, s_act, z, y, ldy, acc=None, stream=None):
    _check(_lib().tern_head_gemv(_ptr(W), _ptr(s_row), _ptr(rowsum), N, K, ldw, M, _ptr(q), ldq,
                                 _ptr(s_act), _ptr(z), _ptr(y), ldy, _ptr(acc), _stream(stream)),
           "tern_head_gemv")


def tern_row_bytes5(K: int) -> int:
    return int(_lib().tern_row_bytes5(int(K)))


def tern_pack5(w, N, K, ldw, packed5, rowsum, bad_count=None, stream=None):
    _check(_lib().tern_pack5(_ptr(w), N, K, ldw, _ptr(packed5), _ptr(rowsum), _ptr(bad_count),
                             _stream(stream)), "tern_pack5")


def tern_gemv5(packed5, s_row, rowsum, N, K, q, s_act, z, y, acc=None, stream=None):
    _check(_lib().tern_gemv5(_ptr(packed5), _ptr(s_row), _ptr(rowsum), N, K, _ptr(q), _ptr(s_act),
                             _ptr(z), _ptr(y), _ptr(acc), _stream(stream)), "tern_gemv5")


def tern_linear_stack_workspace_bytes(L: int, M: int) -> int:
    return int(_lib().tern_linear_stack_workspace_bytes(int(L), int(M)))


def make_desc(packed, s_row, rowsum, N, K, q, ldq, s_act, z, y, ldy, acc=None, block=0, s_block=None,
              rowsum_block=None, x=None, ldx=0, x_up=None) -> tern_linear_desc:
    """One linear of a stack.  With block > 0 (block-wise scales along K),
    s_block / rowsum_block are N x ceil(K / block) and s_row / rowsum may be
    None.  With x (fp32, M x K, row stride ldx) the launch quantises x into
    q, s_act and z itself; with x_up as well, it quantises silu(x) * x_up
    (the gated feed-forward activation; x the gate projection's output)."""
    d = tern_linear_desc()
    d.x = None if x is None else x.data_ptr()
    d.ldx = int(ldx)
    d.x_up = None if x_up is None else x_up.data_ptr()
    d.packed = packed.data_ptr()
    d.s_row = None if s_row is None else s_row.data_ptr()
    d.rowsum = None if rowsum is None else rowsum.data_ptr()
    d.block = int(block)
    d.s_block = None if s_block is None else s_block.data_ptr()
    d.rowsum_block = None if rowsum_block is None else rowsum_block.data_ptr()
    d.N, d.K = int(N), int(K)
    d.q, d.ldq = q.data_ptr(), int(ldq)
    d.s_act, d.z = s_act.data_ptr(), z.data_ptr()
    d.y, d.ldy = y.data_ptr(), int(ldy)
    d.acc = None if acc is None else acc.data_ptr()
    return d


def tern_linear_stack_prepare(descs, M, workspace, path=TERN_PATH_AUTO, stream=None):
    """descs: a sequence of tern_linear_desc; workspace: a device tensor.
    Returns the filled tern_stack_plan (keep it, and the buffers, alive)."""
    arr = (tern_linear_desc * max(1, len(descs)))(*descs)
    plan = tern_stack_plan()
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib().tern_linear_stack_prepare(arr, len(descs), int(M), int(path), _ptr(workspace),
                                            nbytes, ctypes.byref(plan), _stream(stream)),
           "tern_linear_stack_prepare")
    return plan


def tern_linear_stack_prepare_static(descs, M, path=TERN_PATH_AUTO, stream=None):
    """As tern_linear_stack_prepare, with the schedule in the library's own
    device workspace (allocates nothing; the last static prepare on a device
    replaces the schedule of the one before)."""
    arr = (tern_linear_desc * max(1, len(descs)))(*descs)
    plan = tern_stack_plan()
    _check(_lib().tern_linear_stack_prepare_static(arr, len(descs), int(M), int(path), ctypes.byref(plan),
                                                   _stream(stream)),
           "tern_linear_stack_prepare_static")
    return plan


def tern_linear_stack(plan, stream=None):
    _check(_lib().tern_linear_stack(ctypes.byref(plan), _stream(stream)), "tern_linear_stack")


def tern_linear_stack_status(plan, stream=None):
    """Synchronises the stream; raises TernError (TERN_ERR_TIMEOUT) if a
    launch of the plan gave up waiting for a quantised input."""
    _check(_lib().tern_linear_stack_status(ctypes.byref(plan), _stream(stream)), "tern_linear_stack_status")


def tern_read_probe(buf, nbytes, sink, blocks_per_cu=4, unroll=8, nontemporal=True, stream=None):
    _check(_lib().tern_read_probe(_ptr(buf), int(nbytes), _ptr(sink), int(blocks_per_cu),
                                  int(unroll), int(bool(nontemporal)), _stream(stream)),
           "tern_read_probe")
