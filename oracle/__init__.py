"""CPU oracle for the ternary packed-bit linear layer (ctypes over plain C).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.

The C source (``tern_oracle.c``) states what is computed and which passage of
the Neutrino-1 pages each part follows.  This module only compiles it with
``gcc`` and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tern_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libtern_oracle.so")
# -ffp-contract=off: the fp32 output is two separately rounded products.
CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC"]

_lock = threading.Lock()
_lib = None

OK, OVERFLOW, INVALID_CODE = 0, 1, 2


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (always when ``force``)."""
    if (not force and os.path.exists(out)
            and os.path.getmtime(out) >= os.path.getmtime(src)):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _p(t):
    return ctypes.POINTER(t)


def load(path: str | None = None):
    """Load (building first if needed) and type the oracle library."""
    global _lib
    if path is None:
        with _lock:
            if _lib is None:
                _lib = _declare(ctypes.CDLL(build()))
            return _lib
    return _declare(ctypes.CDLL(path))


def _declare(lib):
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_row_bytes.restype = i64
    lib.oracle_row_bytes.argtypes = [i64]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_pack.restype = i64
    lib.oracle_pack.argtypes = [_p(ctypes.c_int8), i64, i64, i64,
                                _p(ctypes.c_uint8), _p(i32)]
    lib.oracle_unpack.restype = i64
    lib.oracle_unpack.argtypes = [_p(ctypes.c_uint8), i64, i64,
                                  _p(ctypes.c_int8), i64]
    lib.oracle_validate.restype = None
    lib.oracle_validate.argtypes = [_p(ctypes.c_uint8), i64, i64, _p(i64)]
    lib.oracle_linear.restype = ctypes.c_int
    lib.oracle_linear.argtypes = [
        _p(ctypes.c_uint8), _p(ctypes.c_float), _p(i32), i64, i64, i64,
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32),
        _p(i32), _p(ctypes.c_float), _p(ctypes.c_double), i64]
    lib.oracle_linear_direct.restype = ctypes.c_int
    lib.oracle_linear_direct.argtypes = [
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), i64, i64, i64,
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32),
        _p(i64), _p(ctypes.c_double), i64]
    lib.oracle_head_rowsum.restype = None
    lib.oracle_head_rowsum.argtypes = [_p(ctypes.c_int8), i64, i64, i64, _p(i32)]
    lib.oracle_head.restype = ctypes.c_int
    lib.oracle_head.argtypes = [
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32), i64, i64, i64,
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32),
        _p(i32), _p(ctypes.c_float), _p(ctypes.c_double), i64]
    lib.oracle_quantize_act.restype = None
    lib.oracle_quantize_act.argtypes = [
        _p(ctypes.c_float), i64, i64, i64, _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32)]
    lib.oracle_block_rowsum.restype = None
    lib.oracle_block_rowsum.argtypes = [_p(ctypes.c_int8), i64, i64, i64, i64, _p(i32)]
    lib.oracle_exp32.restype = None
    lib.oracle_exp32.argtypes = [_p(ctypes.c_float), i64, _p(ctypes.c_float)]
    lib.oracle_swiglu.restype = None
    lib.oracle_swiglu.argtypes = [_p(ctypes.c_float), _p(ctypes.c_float), i64, i64, i64, _p(ctypes.c_float)]
    lib.oracle_linear_blocked.restype = ctypes.c_int
    lib.oracle_linear_blocked.argtypes = [
        _p(ctypes.c_uint8), _p(ctypes.c_float), _p(i32), i64, i64, i64, i64,
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32),
        _p(ctypes.c_float), _p(ctypes.c_double), _p(ctypes.c_double), i64]
    lib.oracle_quantize_weights.restype = None
    lib.oracle_quantize_weights.argtypes = [_p(ctypes.c_float), i64, i64, i64, i64,
                                            _p(ctypes.c_int8), i64, _p(ctypes.c_float)]
    lib.oracle_row_bytes5.restype = i64
    lib.oracle_row_bytes5.argtypes = [i64]
    lib.oracle_pack5.restype = i64
    lib.oracle_pack5.argtypes = [_p(ctypes.c_int8), i64, i64, i64,
                                 _p(ctypes.c_uint8), _p(i32)]
    lib.oracle_unpack5.restype = None
    lib.oracle_unpack5.argtypes = [_p(ctypes.c_uint8), i64, i64, _p(ctypes.c_int8), i64]
    lib.oracle_linear5.restype = ctypes.c_int
    lib.oracle_linear5.argtypes = [
        _p(ctypes.c_uint8), _p(ctypes.c_float), _p(i32), i64, i64, i64,
        _p(ctypes.c_int8), i64, _p(ctypes.c_float), _p(i32),
        _p(i32), _p(ctypes.c_float), _p(ctypes.c_double), i64]
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(_p(ctype))


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def row_bytes(K: int) -> int:
    return int(load().oracle_row_bytes(int(K)))


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's loops from now on (timing only; results do
    not depend on it)."""
    load().oracle_set_threads(int(n))


def pack(w: np.ndarray, lib=None):
    """int8 (N, K) ternary matrix -> (packed uint8 (N, row_bytes), rowsum int32 (N,), bad)."""
    lib = lib or load()
    w = _c(np.atleast_2d(w), np.int8)
    N, K = w.shape
    packed = np.empty((N, row_bytes(K)), np.uint8)
    rowsum = np.empty(N, np.int32)
    bad = lib.oracle_pack(_ptr(w, ctypes.c_int8), N, K, K,
                          _ptr(packed, ctypes.c_uint8), _ptr(rowsum, ctypes.c_int32))
    return packed, rowsum, int(bad)


def unpack(packed: np.ndarray, N: int, K: int, lib=None):
    """Packed rows -> (int8 (N, K) weights, number of invalid 11 fields)."""
    lib = lib or load()
    packed = _c(packed, np.uint8)
    assert packed.size == N * row_bytes(K)
    w = np.empty((N, K), np.int8)
    invalid = lib.oracle_unpack(_ptr(packed, ctypes.c_uint8), N, K,
                                _ptr(w, ctypes.c_int8), K)
    return w, int(invalid)


def validate(packed: np.ndarray, N: int, K: int, lib=None):
    """(invalid 11 fields among real columns, non-01 padding fields)."""
    lib = lib or load()
    packed = _c(packed, np.uint8)
    assert packed.size == N * row_bytes(K)
    counts = np.zeros(2, np.int64)
    lib.oracle_validate(_ptr(packed, ctypes.c_uint8), N, K, _ptr(counts, ctypes.c_int64))
    return int(counts[0]), int(counts[1])


def linear(packed, s_row, rowsum, K, q, s_act, z, lib=None, check=True):
    """acc (int32), y32 (fp32) and y64 (fp64), each (M, N), from packed weights.

    ``q`` is (M, K) int8 (a 1-D vector means M = 1); ``s_act`` and ``z`` hold
    one value per token.
    """
    lib = lib or load()
    q = _c(np.atleast_2d(q), np.int8)
    M = q.shape[0]
    assert q.shape[1] == K
    packed = _c(packed, np.uint8)
    s_row = _c(s_row, np.float32).reshape(-1)
    rowsum = _c(rowsum, np.int32).reshape(-1)
    N = s_row.shape[0]
    assert rowsum.shape[0] == N and packed.size == N * row_bytes(K)
    s_act = _c(np.broadcast_to(np.asarray(s_act, np.float32).reshape(-1), (M,)), np.float32)
    z = _c(np.broadcast_to(np.asarray(z, np.int32).reshape(-1), (M,)), np.int32)
    acc = np.empty((M, N), np.int32)
    y32 = np.empty((M, N), np.float32)
    y64 = np.empty((M, N), np.float64)
    st = lib.oracle_linear(_ptr(packed, ctypes.c_uint8), _ptr(s_row, ctypes.c_float),
                           _ptr(rowsum, ctypes.c_int32), N, K, M,
                           _ptr(q, ctypes.c_int8), K, _ptr(s_act, ctypes.c_float),
                           _ptr(z, ctypes.c_int32), _ptr(acc, ctypes.c_int32),
                           _ptr(y32, ctypes.c_float), _ptr(y64, ctypes.c_double), N)
    if check and st != OK:
        raise ValueError("oracle_linear status %d" % st)
    return acc, y32, y64


def linear_direct(w, s_row, q, s_act, z, lib=None):
    """acc (int64) and y64 (fp64), each (M, N), by sum_j w_ij * (q_mj - z_m)."""
    lib = lib or load()
    w = _c(np.atleast_2d(w), np.int8)
    N, K = w.shape
    q = _c(np.atleast_2d(q), np.int8)
    M = q.shape[0]
    assert q.shape[1] == K
    s_row = _c(s_row, np.float32).reshape(-1)
    s_act = _c(np.broadcast_to(np.asarray(s_act, np.float32).reshape(-1), (M,)), np.float32)
    z = _c(np.broadcast_to(np.asarray(z, np.int32).reshape(-1), (M,)), np.int32)
    acc = np.empty((M, N), np.int64)
    y64 = np.empty((M, N), np.float64)
    lib.oracle_linear_direct(_ptr(w, ctypes.c_int8), K, _ptr(s_row, ctypes.c_float), N, K, M,
                             _ptr(q, ctypes.c_int8), K, _ptr(s_act, ctypes.c_float),
                             _ptr(z, ctypes.c_int32), _ptr(acc, ctypes.c_int64),
                             _ptr(y64, ctypes.c_double), N)
    return acc, y64


def _tokens(q, s_act, z, K):
    q = _c(np.atleast_2d(q), np.int8)
    M = q.shape[0]
    assert q.shape[1] == K
    s_act = _c(np.broadcast_to(np.asarray(s_act, np.float32).reshape(-1), (M,)), np.float32)
    z = _c(np.broadcast_to(np.asarray(z, np.int32).reshape(-1), (M,)), np.int32)
    return q, s_act, z, M


def head_rowsum(W, lib=None):
    """int32 (N,) row sums of an int8 (N, K) output-head matrix."""
    lib = lib or load()
    W = _c(np.atleast_2d(W), np.int8)
    N, K = W.shape
    rowsum = np.empty(N, np.int32)
    lib.oracle_head_rowsum(_ptr(W, ctypes.c_int8), N, K, K, _ptr(rowsum, ctypes.c_int32))
    return rowsum


def head(W, s_row, rowsum, q, s_act, z, lib=None, check=True):
    """Output-head logits: acc (int32), y32 (fp32), y64 (fp64), each (M, N)."""
    lib = lib or load()
    W = _c(np.atleast_2d(W), np.int8)
    N, K = W.shape
    q, s_act, z, M = _tokens(q, s_act, z, K)
    s_row = _c(s_row, np.float32).reshape(-1)
    rowsum = _c(rowsum, np.int32).reshape(-1)
    assert s_row.shape[0] == N and rowsum.shape[0] == N
    acc = np.empty((M, N), np.int32)
    y32 = np.empty((M, N), np.float32)
    y64 = np.empty((M, N), np.float64)
    st = lib.oracle_head(_ptr(W, ctypes.c_int8), K, _ptr(s_row, ctypes.c_float),
                         _ptr(rowsum, ctypes.c_int32), N, K, M, _ptr(q, ctypes.c_int8), K,
                         _ptr(s_act, ctypes.c_float), _ptr(z, ctypes.c_int32),
                         _ptr(acc, ctypes.c_int32), _ptr(y32, ctypes.c_float),
                         _ptr(y64, ctypes.c_double), N)
    if check and st != OK:
        raise ValueError("oracle_head status %d" % st)
    return acc, y32, y64


def quantize_act(x, lib=None):
    """Per-token asymmetric int8: x (M, K) float32 -> (q int8 (M, K), s_act (M,), z (M,))."""
    lib = lib or load()
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s_act = np.empty(M, np.float32)
    z = np.empty(M, np.int32)
    lib.oracle_quantize_act(_ptr(x, ctypes.c_float), M, K, K, _ptr(q, ctypes.c_int8), K,
                            _ptr(s_act, ctypes.c_float), _ptr(z, ctypes.c_int32))
    return q, s_act, z


def exp32(x, lib=None):
    """The fp32 exp of the SwiGLU evaluation (Cody-Waite reduction, Taylor to
    r^7): float32 array of the same shape."""
    lib = lib or load()
    x = _c(np.asarray(x), np.float32)
    out = np.empty_like(x)
    lib.oracle_exp32(_ptr(x, ctypes.c_float), x.size, _ptr(out, ctypes.c_float))
    return out


def swiglu(g, u, lib=None):
    """h = silu(g) * u in the fixed fp32 steps of oracle_swiglu (model card
    "Neutrino-1 8B", "Architecture": gated SwiGLU feed-forward); (M, K)."""
    lib = lib or load()
    g = _c(np.atleast_2d(g), np.float32)
    u = _c(np.atleast_2d(u), np.float32)
    assert g.shape == u.shape
    M, K = g.shape
    h = np.empty((M, K), np.float32)
    lib.oracle_swiglu(_ptr(g, ctypes.c_float), _ptr(u, ctypes.c_float), M, K, K, _ptr(h, ctypes.c_float))
    return h


def block_rowsum(w, B, lib=None):
    """int32 (N, ceil(K / B)) per-block row sums of an int8 ternary (N, K) matrix."""
    lib = lib or load()
    w = _c(np.atleast_2d(w), np.int8)
    N, K = w.shape
    nb = (K + B - 1) // B
    out = np.empty((N, nb), np.int32)
    lib.oracle_block_rowsum(_ptr(w, ctypes.c_int8), N, K, K, B, _ptr(out, ctypes.c_int32))
    return out


def linear_blocked(packed, s_b, rowsum_b, K, B, q, s_act, z, lib=None, check=True):
    """Block-scaled linear: y32 (reference fp32 order), y64, yabs, each (M, N)."""
    lib = lib or load()
    q, s_act, z, M = _tokens(q, s_act, z, K)
    packed = _c(packed, np.uint8)
    s_b = _c(np.atleast_2d(s_b), np.float32)
    rowsum_b = _c(np.atleast_2d(rowsum_b), np.int32)
    N, nb = s_b.shape
    assert nb == (K + B - 1) // B and rowsum_b.shape == (N, nb)
    assert packed.size == N * row_bytes(K)
    y32 = np.empty((M, N), np.float32)
    y64 = np.empty((M, N), np.float64)
    yabs = np.empty((M, N), np.float64)
    st = lib.oracle_linear_blocked(_ptr(packed, ctypes.c_uint8), _ptr(s_b, ctypes.c_float),
                                   _ptr(rowsum_b, ctypes.c_int32), N, K, B, M,
                                   _ptr(q, ctypes.c_int8), K, _ptr(s_act, ctypes.c_float),
                                   _ptr(z, ctypes.c_int32), _ptr(y32, ctypes.c_float),
                                   _ptr(y64, ctypes.c_double), _ptr(yabs, ctypes.c_double), N)
    if check and st != OK:
        raise ValueError("oracle_linear_blocked status %d" % st)
    return y32, y64, yabs


def quantize_weights(W, B, lib=None):
    """fp32 (N, K) weights -> (states int8 (N, K), block scales fp32 (N, ceil(K / B)))."""
    lib = lib or load()
    W = _c(np.atleast_2d(W), np.float32)
    N, K = W.shape
    nb = (K + B - 1) // B
    t = np.empty((N, K), np.int8)
    s_b = np.empty((N, nb), np.float32)
    lib.oracle_quantize_weights(_ptr(W, ctypes.c_float), N, K, K, int(B), _ptr(t, ctypes.c_int8), K,
                                _ptr(s_b, ctypes.c_float))
    return t, s_b


# ---- 1.6-bit rows (five weights per byte) ----

def row_bytes5(K: int, lib=None) -> int:
    return int((lib or load()).oracle_row_bytes5(int(K)))


def pack5(w, lib=None):
    """int8 (N, K) ternary matrix -> (1.6-bit rows uint8 (N, row_bytes5), rowsum int32 (N,), bad)."""
    lib = lib or load()
    w = _c(np.atleast_2d(w), np.int8)
    N, K = w.shape
    packed = np.empty((N, row_bytes5(K, lib)), np.uint8)
    rowsum = np.empty(N, np.int32)
    bad = lib.oracle_pack5(_ptr(w, ctypes.c_int8), N, K, K,
                           _ptr(packed, ctypes.c_uint8), _ptr(rowsum, ctypes.c_int32))
    return packed, rowsum, int(bad)


def unpack5(packed, N: int, K: int, lib=None):
    """1.6-bit rows -> int8 (N, K) weights (every byte decodes)."""
    lib = lib or load()
    packed = _c(packed, np.uint8)
    assert packed.size == N * row_bytes5(K, lib)
    w = np.empty((N, K), np.int8)
    lib.oracle_unpack5(_ptr(packed, ctypes.c_uint8), N, K, _ptr(w, ctypes.c_int8), K)
    return w


def linear5(packed, s_row, rowsum, K, q, s_act, z, lib=None, check=True):
    """The linear layer on 1.6-bit rows: acc (int32), y32, y64, each (M, N)."""
    lib = lib or load()
    q, s_act, z, M = _tokens(q, s_act, z, K)
    packed = _c(packed, np.uint8)
    s_row = _c(s_row, np.float32).reshape(-1)
    rowsum = _c(rowsum, np.int32).reshape(-1)
    N = s_row.shape[0]
    assert rowsum.shape[0] == N and packed.size == N * row_bytes5(K, lib)
    acc = np.empty((M, N), np.int32)
    y32 = np.empty((M, N), np.float32)
    y64 = np.empty((M, N), np.float64)
    st = lib.oracle_linear5(_ptr(packed, ctypes.c_uint8), _ptr(s_row, ctypes.c_float),
                            _ptr(rowsum, ctypes.c_int32), N, K, M, _ptr(q, ctypes.c_int8), K,
                            _ptr(s_act, ctypes.c_float), _ptr(z, ctypes.c_int32),
                            _ptr(acc, ctypes.c_int32), _ptr(y32, ctypes.c_float),
                            _ptr(y64, ctypes.c_double), N)
    if check and st != OK:
        raise ValueError("oracle_linear5 status %d" % st)
    return acc, y32, y64
