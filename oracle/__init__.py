"""CPU oracle for the dense-GEMM path.  TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does, and this package never imports the
GPU library.  The arithmetic lives in ``oracle.c`` (binary64, plain loops);
this module only marshals numpy arrays into it.

Pinned by ``tests/test_oracle_*.py`` against brute force in exact rational
arithmetic, integer triple loops, identity/permutation products, closed forms
and numpy's float16 cast.  The tanh-GELU epilogue has no value printed on the
pages to pin it; it is pinned by its exact special cases (GELU(0) = 0, the
odd symmetry of its tanh argument, the limits x and 0 for large |x|) and by
an independent evaluation through the error function's relation
(see ``tests/test_oracle_epilogue.py``).

``dequant("q4_k", ...)`` is PARITY UNPINNED: the pages name the q4_K type but
print no layout, so the super-block layout it decodes is a reading from
outside them, and its golden blocks follow the same reading.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, F32 = 0, 1, 2
_TYPES = {"f16": F16, "bf16": BF16, "f32": F32}
_BITS = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}
EPI = {"none": 0, "bias": 1, "bias_gelu": 2}

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        i64, dbl, vp, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = dbl
        L.oracle_f64_to_f16.argtypes = [dbl]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [dbl]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_f64_to_f32.argtypes = [dbl]
        L.oracle_f64_to_f32.restype = ctypes.c_uint32
        L.oracle_gelu_tanh.argtypes = [dbl]
        L.oracle_gelu_tanh.restype = dbl
        L.oracle_decode.argtypes = [i32, i64, vp, vp]
        L.oracle_decode.restype = None
        L.oracle_encode.argtypes = [i32, i64, vp, vp]
        L.oracle_encode.restype = None
        L.oracle_gemm.argtypes = [i64, i64, i64, dbl, i32, vp, i64, i32, vp, i64, i32, dbl,
                                  vp, i64, i32, vp, vp, vp, i32]
        L.oracle_gemm.restype = i32
        L.oracle_dequant_q4.argtypes = [vp, i64, i64, vp, i64]
        L.oracle_dequant_q4.restype = i32
        L.oracle_dequant_q6_k.argtypes = [vp, i64, i64, i64, vp, i64]
        L.oracle_dequant_q6_k.restype = i32
        L.oracle_dequant_q4_k.argtypes = [vp, i64, i64, vp, i64]
        L.oracle_dequant_q4_k.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(bits, dtype):
    """Raw bits (uint16 for f16/bf16, uint32 for f32) -> exact float64 values."""
    bits = np.ascontiguousarray(bits, dtype=_BITS[dtype])
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_decode(_TYPES[dtype], bits.size, _ptr(bits), _ptr(out))
    return out


def encode(x, dtype):
    """float64 values -> raw bits of dtype, rounded to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=_BITS[dtype])
    lib().oracle_encode(_TYPES[dtype], x.size, _ptr(x), _ptr(out))
    return out


def gelu_tanh(t):
    return lib().oracle_gelu_tanh(float(t))


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def gemm(A, B, dtype, trans_b=False, alpha=1.0, beta=0.0, C_old=None, epi="none", bias=None,
         want_U=True, threads=None):
    """Binary64 reference of epi(alpha*A@B + beta*C_old).

    A: (M, K) raw bits of ``dtype``; B: (K, N) raw bits, or (N, K) when
    ``trans_b``.  C_old and bias are binary64 values (decode them first).
    Returns (T, U): T the binary64 result before output rounding, U the
    elementwise scale sum_k |A_ik||B_kj| (None if not wanted).
    """
    A = np.ascontiguousarray(A, dtype=_BITS[dtype])
    B = np.ascontiguousarray(B, dtype=_BITS[dtype])
    M, K = A.shape
    if trans_b:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, Kb))
    out = np.zeros((M, N), dtype=np.float64)
    U = np.zeros((M, N), dtype=np.float64) if want_U else None
    cin = None
    if beta != 0.0:
        cin = np.ascontiguousarray(C_old, dtype=np.float64)
        assert cin.shape == (M, N)
    b = None
    if EPI[epi] != 0:
        b = np.ascontiguousarray(bias, dtype=np.float64)
        assert b.shape == (N,)
    rc = lib().oracle_gemm(M, N, K, float(alpha), _TYPES[dtype], _ptr(A), K, _TYPES[dtype],
                           _ptr(B), B.shape[1], 1 if trans_b else 0, float(beta), _ptr(cin), N,
                           EPI[epi], _ptr(b), _ptr(out), _ptr(U),
                           threads or default_threads())
    if rc != 0:
        raise MemoryError("oracle_gemm failed")
    return out, U


def dequant_q4(q, rows, cols):
    """Raw q4 blocks (uint8, rows*cols/32*18 bytes) -> (rows, cols) binary16 bits."""
    q = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1)
    if cols % 32 != 0:
        raise ValueError("cols must be a multiple of 32")
    if q.size != rows * (cols // 32) * 18:
        raise ValueError("expected %d bytes, got %d" % (rows * (cols // 32) * 18, q.size))
    out = np.empty((rows, cols), dtype=np.uint16)
    rc = lib().oracle_dequant_q4(_ptr(q), rows, cols, _ptr(out), cols)
    if rc != 0:
        raise ValueError("oracle_dequant_q4 rejected the shape")
    return out


# weights and bytes per block; "q6_k_224" is q6_K at a 224-byte block stride
QTYPES = {"q4_0": (32, 18), "q4_k": (256, 144), "q6_k": (256, 210), "q6_k_224": (256, 224)}


def dequant(qtype, q, rows, cols):
    """Raw blocks of a weight type ("q4_0", "q4_k", "q6_k", "q6_k_224") ->
    (rows, cols) binary16 bits."""
    if qtype == "q4_0":
        return dequant_q4(q, rows, cols)
    per, nbytes = QTYPES[qtype]
    q = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1)
    if cols % per != 0:
        raise ValueError("cols must be a multiple of %d" % per)
    if q.size != rows * (cols // per) * nbytes:
        raise ValueError("expected %d bytes, got %d" % (rows * (cols // per) * nbytes, q.size))
    out = np.empty((rows, cols), dtype=np.uint16)
    if qtype.startswith("q6_k"):
        st = lib().oracle_dequant_q6_k(_ptr(q), rows, cols, nbytes, _ptr(out), cols)
    else:
        st = lib().oracle_dequant_q4_k(_ptr(q), rows, cols, _ptr(out), cols)
    if st != 0:
        raise ValueError("dequant rejected the shape")
    return out


def prefill(A, q, N, K, want_U=True, threads=None):
    """Prefill projection: C = A @ W16^T with W16 the oracle dequant of q (N x K)."""
    W16 = dequant_q4(q, N, K)
    T, U = gemm(A, W16, "f16", trans_b=True, want_U=want_U, threads=threads)
    return T, U, W16
