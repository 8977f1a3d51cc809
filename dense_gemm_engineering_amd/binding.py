"""Thin Python binding over the C ABI in include/gemm.h.

Argument marshalling only: torch tensors supply device memory and the
stream; every step runs in the gfx950 kernels of libdge_gemm.so.  If the
library is missing, loading fails loudly (there is no fallback path).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdge_gemm.so")
# the diagnostic build of the same library (extra waits and barriers in the
# direct-to-LDS kernels); only tests select it, through diag_library()
LIB_DIAG_PATH = os.path.join(_HERE, "libdge_gemm_diag.so")

GEMM_OK = 0
STATUS_NAMES = {0: "GEMM_OK", 1: "GEMM_ERR_INVALID_VALUE", 2: "GEMM_ERR_NOT_SUPPORTED",
                3: "GEMM_ERR_WORKSPACE", 4: "GEMM_ERR_LAUNCH", 5: "GEMM_ERR_DEVICE",
                6: "GEMM_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20
EPI = {"none": 0, "bias": 1, "bias_gelu": 2}
OUT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
IN = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}
ALGO = {"auto": 0, "naive": 1, "lds_tiled": 2, "mfma": 3, "mfma_direct": 4, "skinny": 5,
        "decode": 6, "streamk": 7}
TILE = {"auto": 0, "256x256": 1, "256x128": 2, "128x128": 3, "128x64": 4, "256x256w8": 5, "256x128w8": 6}
QTYPE = {"q4_0": 0, "q4_k": 1, "q6_k": 2, "q6_k_224": 3}

# Every symbol include/gemm.h declares.
EXPORTS = ("gemm_f16", "gemm_bf16", "gemm_f32", "gemm_ex", "gemm_ex_noalloc", "dequant_q4_f16",
           "prefill_q4_f16",
           "gemm_q4_f16", "dequant_f16", "prefill_f16",
           "gemm_workspace_size", "gemm_workspace_size_splits", "gemm_workspace_size_streamk",
           "gemm_status_string", "gemm_init",
           # measurement probes (include/gemm_probe.h)
           "gemm_probe_clock", "gemm_probe_phases", "gemm_probe_mfma", "gemm_probe_read",
           "gemm_probe_copy")
PROBE_MFMA_GRID = 256


class GemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, gemm_status_string(status)))


class Tuning(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int), ("tile", ctypes.c_int), ("splits", ctypes.c_int)]


_libs = {}
_active = [LIB_PATH]


class diag_library:
    """Context manager: calls inside it go to the diagnostic build."""

    def __enter__(self):
        _active.append(LIB_DIAG_PATH)
        return self

    def __exit__(self, *exc):
        _active.pop()
        return False


def lib():
    """Load libdge_gemm.so (raises if it has not been built)."""
    path = _active[-1]
    if path not in _libs:
        if not os.path.exists(path):
            raise ImportError("%s is not built (run __graft_entry__.build())" % path)
        L = ctypes.CDLL(path)
        i64, f32, vp, i32, sz = (ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_size_t)
        gemm_args = [i64, i64, i64, f32, vp, i64, vp, i64, i32, f32, vp, i64, i32, i32, vp, vp, sz,
                     vp]
        for name in ("gemm_f16", "gemm_bf16", "gemm_f32"):
            fn = getattr(L, name)
            fn.argtypes = gemm_args
            fn.restype = i32
        L.gemm_ex.argtypes = [i32] + gemm_args[:-1] + [ctypes.POINTER(Tuning), vp]
        L.gemm_ex.restype = i32
        L.gemm_ex_noalloc.argtypes = [i32] + gemm_args[:-3] + [ctypes.POINTER(Tuning), vp]
        L.gemm_ex_noalloc.restype = i32
        L.dequant_q4_f16.argtypes = [vp, vp, i64, i64, i64, vp]
        L.dequant_q4_f16.restype = i32
        L.prefill_q4_f16.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, i64, i32, i32, vp, vp, sz,
                                     vp]
        L.prefill_q4_f16.restype = i32
        L.gemm_q4_f16.argtypes = [i64, i64, i64, vp, i64, vp, vp, i64, i32, i32, vp, vp, sz,
                                  ctypes.POINTER(Tuning), vp]
        L.gemm_q4_f16.restype = i32
        L.dequant_f16.argtypes = [i32, vp, vp, i64, i64, i64, vp]
        L.dequant_f16.restype = i32
        L.prefill_f16.argtypes = [i32] + L.prefill_q4_f16.argtypes
        L.prefill_f16.restype = i32
        L.gemm_workspace_size.argtypes = [i64, i64, i64, i32]
        L.gemm_workspace_size.restype = sz
        L.gemm_workspace_size_splits.argtypes = [i64, i64, i32]
        L.gemm_workspace_size_splits.restype = sz
        L.gemm_workspace_size_streamk.argtypes = [i64, i64, i64, i32]
        L.gemm_workspace_size_streamk.restype = sz
        L.gemm_status_string.argtypes = [i32]
        L.gemm_status_string.restype = ctypes.c_char_p
        L.gemm_init.argtypes = []
        L.gemm_init.restype = i32
        L.gemm_probe_clock.argtypes = [i32] + gemm_args[:-3] + [vp, i64, vp]
        L.gemm_probe_clock.restype = i32
        L.gemm_probe_phases.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, i32, vp, i64, i32,
                                        i32, vp, vp, sz, vp, i64, vp]
        L.gemm_probe_phases.restype = i32
        L.gemm_probe_mfma.argtypes = [i32, vp, i64, vp, i64, i64, i64, i32, vp, vp, vp]
        L.gemm_probe_mfma.restype = i32
        L.gemm_probe_read.argtypes = [vp, sz, i32, vp, vp]
        L.gemm_probe_read.restype = i32
        L.gemm_probe_copy.argtypes = [vp, vp, sz, i32, vp]
        L.gemm_probe_copy.restype = i32
        _libs[path] = L
    return _libs[path]


def gemm_status_string(status):
    return lib().gemm_status_string(int(status)).decode()


def _check(status, where):
    if status != GEMM_OK:
        raise GemmError(status, where)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t, name):
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major (unit column stride)" % name)
    return max(t.stride(0), t.size(1), 1)


def _prepare(A, B, C, trans_b, out_dtype):
    M, K = A.shape
    if trans_b:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, Kb))
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError("C has shape %s, expected %s" % (tuple(C.shape), (M, N)))
    return M, N, K, C


def _gemm_call(fn_name, A, B, C, trans_b, alpha, beta, out_dtype, epi, bias, workspace, stream,
               tuning=None):
    M, N, K, C = _prepare(A, B, C, trans_b, out_dtype)
    args = [M, N, K, float(alpha), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"), int(bool(trans_b)),
            float(beta), _ptr(C), _ld(C, "C"), OUT[C.dtype], EPI[epi], _ptr(bias),
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()]
    L = lib()
    if fn_name == "gemm_ex_noalloc":
        st = L.gemm_ex_noalloc(IN[A.dtype], *args[:-2],
                               ctypes.byref(tuning) if tuning is not None else None,
                               _stream(stream))
    elif fn_name == "gemm_ex":
        st = L.gemm_ex(IN[A.dtype], *args, ctypes.byref(tuning) if tuning is not None else None,
                       _stream(stream))
    else:
        st = getattr(L, fn_name)(*args, _stream(stream))
    _check(st, fn_name)
    return C


def gemm_f16(A, B, C=None, *, trans_b=False, alpha=1.0, beta=0.0, out_dtype=torch.float16,
             epi="none", bias=None, workspace=None, stream=None):
    """C = epi(alpha * A @ B + beta * C) with fp16 A, B (B is N x K when trans_b)."""
    return _gemm_call("gemm_f16", A, B, C, trans_b, alpha, beta, out_dtype, epi, bias, workspace,
                      stream)


def gemm_bf16(A, B, C=None, *, trans_b=False, alpha=1.0, beta=0.0, out_dtype=torch.float16,
              epi="none", bias=None, workspace=None, stream=None):
    return _gemm_call("gemm_bf16", A, B, C, trans_b, alpha, beta, out_dtype, epi, bias, workspace,
                      stream)


def gemm_f32(A, B, C=None, *, trans_b=False, alpha=1.0, beta=0.0, out_dtype=torch.float32,
             epi="none", bias=None, workspace=None, stream=None):
    return _gemm_call("gemm_f32", A, B, C, trans_b, alpha, beta, out_dtype, epi, bias, workspace,
                      stream)


def gemm_ex(A, B, C=None, *, trans_b=False, alpha=1.0, beta=0.0, out_dtype=None, epi="none",
            bias=None, workspace=None, algo="auto", tile="auto", splits=0, stream=None):
    """The same operation with the kernel family, tile and split chosen explicitly."""
    if out_dtype is None:
        out_dtype = torch.float32 if A.dtype == torch.float32 else torch.float16
    t = Tuning(ALGO[algo], TILE[tile], int(splits))
    return _gemm_call("gemm_ex", A, B, C, trans_b, alpha, beta, out_dtype, epi, bias, workspace,
                      stream, tuning=t)


def gemm_ex_noalloc(A, B, C=None, *, trans_b=False, alpha=1.0, beta=0.0, out_dtype=None,
                    epi="none", bias=None, algo="auto", tile="auto", splits=0, stream=None):
    """gemm_ex with the library's static scratch in place of a workspace (the
    call allocates nothing; calls overlapping on one device race)."""
    if out_dtype is None:
        out_dtype = torch.float32 if A.dtype == torch.float32 else torch.float16
    t = Tuning(ALGO[algo], TILE[tile], int(splits))
    return _gemm_call("gemm_ex_noalloc", A, B, C, trans_b, alpha, beta, out_dtype, epi, bias,
                      None, stream, tuning=t)


def gemm(A, B, C=None, **kw):
    """Dispatch on A's dtype to gemm_f16 / gemm_bf16 / gemm_f32."""
    fn = {torch.float16: gemm_f16, torch.bfloat16: gemm_bf16, torch.float32: gemm_f32}[A.dtype]
    return fn(A, B, C, **kw)


def dequant_q4_f16(q, rows, cols, out=None, stream=None):
    """q: uint8 device tensor of rows*cols/32*18 bytes -> (rows, cols) fp16."""
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=q.device)
    ldo = _ld(out, "out") if out.numel() else cols
    _check(lib().dequant_q4_f16(_ptr(q), _ptr(out), rows, cols, ldo, _stream(stream)),
           "dequant_q4_f16")
    return out


def prefill_q4_f16(A, q, N, K, w16=None, C=None, *, out_dtype=torch.float16, epi="none",
                   bias=None, workspace=None, stream=None):
    """C = epi(A @ dequant(q)^T); w16 is the caller's fp16 N x K scratch."""
    M = A.shape[0]
    if w16 is None:
        w16 = torch.empty((N, K), dtype=torch.float16, device=A.device)
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().prefill_q4_f16(M, N, K, _ptr(A), _ld(A, "A"), _ptr(q), _ptr(w16), _ptr(C),
                                _ld(C, "C"), OUT[C.dtype], EPI[epi], _ptr(bias), _ptr(workspace),
                                ws_bytes, _stream(stream)), "prefill_q4_f16")
    return C


def dequant_f16(qtype, q, rows, cols, out=None, stream=None):
    """q: uint8 device tensor of blocks in format qtype ("q4_0", "q4_k",
    "q6_k", "q6_k_224") -> (rows, cols) fp16."""
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=q.device)
    ldo = _ld(out, "out") if out.numel() else cols
    _check(lib().dequant_f16(QTYPE[qtype], _ptr(q), _ptr(out), rows, cols, ldo, _stream(stream)),
           "dequant_f16")
    return out


def prefill_f16(qtype, A, q, N, K, w16=None, C=None, *, out_dtype=torch.float16, epi="none",
                bias=None, workspace=None, stream=None):
    """C = epi(A @ dequant_f16(qtype, q)^T); w16 is the caller's fp16 N x K scratch."""
    M = A.shape[0]
    if w16 is None:
        w16 = torch.empty((N, K), dtype=torch.float16, device=A.device)
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().prefill_f16(QTYPE[qtype], M, N, K, _ptr(A), _ld(A, "A"), _ptr(q), _ptr(w16),
                             _ptr(C), _ld(C, "C"), OUT[C.dtype], EPI[epi], _ptr(bias),
                             _ptr(workspace), ws_bytes, _stream(stream)), "prefill_f16")
    return C


def gemm_q4_f16(A, q, N, K, C=None, *, out_dtype=torch.float16, epi="none", bias=None,
                workspace=None, algo="auto", tile="auto", splits=0, stream=None):
    """C = epi(A @ dequant(q)^T) with the dequantisation fused into the GEMM
    (algo="mfma_direct" requires the fused kernel)."""
    M = A.shape[0]
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    t = Tuning(ALGO[algo], TILE[tile], int(splits))
    _check(lib().gemm_q4_f16(M, N, K, _ptr(A), _ld(A, "A"), _ptr(q), _ptr(C), _ld(C, "C"),
                             OUT[C.dtype], EPI[epi], _ptr(bias), _ptr(workspace), ws_bytes,
                             ctypes.byref(t), _stream(stream)), "gemm_q4_f16")
    return C


def probe_clock(A, B, C, clk, *, trans_b=False, stream=None):
    """The automatic GEMM C = A @ B (one data-parallel launch) with clock
    records: clk is a uint64 (int64) device tensor of 4 values per workgroup."""
    M, N, K, C = _prepare(A, B, C, trans_b, C.dtype)
    _check(lib().gemm_probe_clock(IN[A.dtype], M, N, K, 1.0, _ptr(A), _ld(A, "A"), _ptr(B),
                                  _ld(B, "B"), int(bool(trans_b)), 0.0, _ptr(C), _ld(C, "C"),
                                  OUT[C.dtype], 0, None, _ptr(clk), clk.numel() // 4,
                                  _stream(stream)), "gemm_probe_clock")
    return C


def probe_phases(A, B, C, rec, *, trans_b=False, epi="none", bias=None, workspace=None,
                 stream=None):
    """The automatic GEMM with phase records (the split decode schedule):
    rec is an int64 device tensor of 4 real-time counter values per
    workgroup."""
    M, N, K, C = _prepare(A, B, C, trans_b, C.dtype)
    _check(lib().gemm_probe_phases(IN[A.dtype], M, N, K, _ptr(A), _ld(A, "A"), _ptr(B),
                                   _ld(B, "B"), int(bool(trans_b)), _ptr(C), _ld(C, "C"),
                                   OUT[C.dtype], EPI[epi], _ptr(bias), _ptr(workspace),
                                   0 if workspace is None else
                                   workspace.numel() * workspace.element_size(),
                                   _ptr(rec), rec.numel() // 4,
                                   _stream(stream)), "gemm_probe_phases")
    return C


def probe_mfma(A, B, k_blocks, out, clk=None, stream=None):
    """MFMA-only probe over operand fragments of A and B (>= 4096 rows)."""
    _check(lib().gemm_probe_mfma(IN[A.dtype], _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"),
                                 min(A.shape[0], B.shape[0]), min(A.shape[1], B.shape[1]),
                                 int(k_blocks), _ptr(out), _ptr(clk), _stream(stream)),
           "gemm_probe_mfma")


def probe_read(src, out, grid, stream=None):
    """Streaming read of src on `grid` workgroups; out: >= grid x 256 int32."""
    assert out.numel() >= grid * 256
    _check(lib().gemm_probe_read(_ptr(src), src.numel() * src.element_size(), int(grid),
                                 _ptr(out), _stream(stream)), "gemm_probe_read")


def probe_copy(src, dst, grid, stream=None):
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    _check(lib().gemm_probe_copy(_ptr(src), _ptr(dst), n, int(grid), _stream(stream)),
           "gemm_probe_copy")


def gemm_workspace_size(M, N, K, dtype=torch.float16):
    return lib().gemm_workspace_size(M, N, K, IN[dtype])


def gemm_workspace_size_splits(M, N, splits):
    return lib().gemm_workspace_size_splits(M, N, splits)


def gemm_workspace_size_streamk(M, N, K, tile="auto"):
    return lib().gemm_workspace_size_streamk(M, N, K, TILE[tile])


def gemm_init():
    _check(lib().gemm_init(), "gemm_init")
