"""Helpers for the GPU parity tests: host bits <-> device tensors, checks."""
import numpy as np
import torch

import oracle
from oracle import compare

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
OUT_NAME = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}


def to_dev(bits, dtype):
    """Raw host bits (uint16 / uint32 numpy) -> device tensor of dtype name."""
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(bits.view(np.int32).copy()).view(torch.float32)
    else:
        t = torch.from_numpy(bits.view(np.int16).copy()).view(TORCH_DT[dtype])
    return t.cuda()


def bits_of(t):
    """Device/host tensor -> raw host bits (uint16 for 16-bit types, uint32 for fp32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def values_of(t):
    """Device tensor -> exact float64 host values (decoded by the oracle)."""
    return oracle.decode(bits_of(t), OUT_NAME[t.dtype])


def assert_close(C, T, U, alpha=1.0, beta=0.0, C_old=None, bias=None, what=""):
    scale = compare.elem_scale(U, alpha, beta, C_old, bias)
    ok, rep = compare.check_tolerance(values_of(C), T, scale,
                                      compare.normwise_tol(OUT_NAME[C.dtype]))
    assert ok, "%s: %s" % (what, rep)
    return rep


def assert_bits(C, T, what=""):
    want = oracle.encode(T, OUT_NAME[C.dtype])
    got = bits_of(C)
    n = compare.bits_mismatch(got, want)
    if n:
        idx = np.argwhere(got != want)[:5]
        detail = [(tuple(i), int(got[tuple(i)]), int(want[tuple(i)]), T[tuple(i)]) for i in idx]
        raise AssertionError("%s: %d elements differ in bits; first %s" % (what, n, detail))


def sample_rows(M, n, seed=0):
    r = np.random.Generator(np.random.PCG64(seed))
    rows = np.sort(r.choice(M, size=min(n, M), replace=False))
    # always include the first and last row (tile edges)
    return np.unique(np.concatenate([[0, M - 1], rows]))
