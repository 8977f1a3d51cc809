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


def assert_close(C, T, U, alpha=1.0, what=""):
    """C within the acceptance bounds of the oracle's T: normwise, and every
    element within 1e-2 |alpha| U_ij + 1e-3.  The bound must first admit the
    oracle's own correctly rounded result with room to spare (else the test
    input, not the kernel, is at fault)."""
    out = OUT_NAME[C.dtype]
    scale = compare.elem_scale(U, alpha)
    assert compare.rounding_fits(oracle.decode(oracle.encode(T, out), out), T, scale), \
        "%s: the bound does not admit the rounded exact result" % what
    got = values_of(C)
    ok, rep = compare.check_tolerance(got, T, scale, compare.normwise_tol(out))
    if not ok:
        bad = np.argwhere(~(np.abs(got - T) <= compare.ELEM_RTOL * scale + compare.ELEM_ATOL))[:5]
        rep["first_bad"] = [(tuple(int(x) for x in i), float(got[tuple(i)]), float(T[tuple(i)]),
                             float(scale[tuple(i)])) for i in bad]
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

