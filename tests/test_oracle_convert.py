"""Pins for the oracle's number-format conversions.

Decoders are checked on every bit pattern against numpy (float16) and torch
(bfloat16), encoders at every representable value, every midpoint between
neighbours and the floating-point neighbours of those midpoints against the
library casts, which round to nearest, ties to even.
"""
import numpy as np
import pytest
import torch

import oracle

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _same_or_both_nan(a, b):
    return np.all((a == b) | (np.isnan(a) & np.isnan(b)))


def test_decode_f16_all_patterns():
    got = oracle.decode(ALL16, "f16")
    want = ALL16.view(np.float16).astype(np.float64)
    assert _same_or_both_nan(got, want)
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_decode_bf16_all_patterns():
    got = oracle.decode(ALL16, "bf16")
    want = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same_or_both_nan(got, want)


def test_decode_f32_sample_and_specials():
    r = np.random.Generator(np.random.PCG64(7))
    bits = r.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x807fffff, 0x00800000, 0x7f7fffff, 0x7f800000,
                         0xff800000, 0x3f800000, 0x7fc00000], dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    got = oracle.decode(bits, "f32")
    want = bits.view(np.float32).astype(np.float64)
    assert _same_or_both_nan(got, want)


def _finite16(decoded):
    return np.unique(decoded[np.isfinite(decoded)])


def _midpoints_and_neighbours(vals):
    vals = np.sort(vals)
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in binary64 for 16-bit formats
    nb = np.concatenate([np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    return np.concatenate([vals, mids, nb])


def test_encode_f16_exhaustive_midpoints():
    vals = _finite16(ALL16.view(np.float16).astype(np.float64))
    xs = _midpoints_and_neighbours(vals)
    # beyond the largest finite value: the overflow boundary 65520 and above
    xs = np.concatenate([xs, [65519.999, 65520.0, 65536.0, 1e10, -65520.0, np.inf, -np.inf,
                              2.0**-25, -2.0**-25, 2.0**-26, 3 * 2.0**-26, 1e-30]])
    got = oracle.encode(xs, "f16")
    want = xs.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], got[i], want[i]) for i in bad[:10]]


def test_encode_f16_random_doubles():
    r = np.random.Generator(np.random.PCG64(11))
    xs = r.standard_normal(500000) * np.exp2(r.integers(-30, 18, size=500000))
    got = oracle.encode(xs, "f16")
    want = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_exhaustive_midpoints():
    # bf16 values, their midpoints and the float32 neighbours of the midpoints
    # are all float32 numbers, where torch's float32 -> bfloat16 cast is a
    # single round-to-nearest-even.
    dec = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    vals = np.unique(dec[np.isfinite(dec)]).astype(np.float64)
    vals = np.sort(vals)
    mids = ((vals[:-1] + vals[1:]) / 2.0).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2.0)
    nb = np.concatenate([np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    xs32 = np.concatenate([vals.astype(np.float32), mids, nb,
                           np.array([3.0e38, -3.4e38, np.inf, -np.inf], dtype=np.float32)])
    got = oracle.encode(xs32.astype(np.float64), "bf16")
    want = torch.from_numpy(xs32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs32[i], got[i], want[i]) for i in bad[:10]]


def test_encode_f32_midpoints():
    r = np.random.Generator(np.random.PCG64(13))
    a = (r.standard_normal(200000) * np.exp2(r.integers(-140, 120, size=200000))).astype(np.float32)
    b = np.nextafter(a, np.float32(np.inf))
    mids = (a.astype(np.float64) + b.astype(np.float64)) / 2.0
    xs = np.concatenate([a.astype(np.float64), mids, np.nextafter(mids, np.inf),
                         np.nextafter(mids, -np.inf), [3.5e38, -3.5e38, 1e-46, 7e-46]])
    xs = xs[np.isfinite(xs)]
    got = oracle.encode(xs, "f32")
    want = xs.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_roundtrip_all_finite(dtype):
    if dtype == "f32":
        r = np.random.Generator(np.random.PCG64(17))
        bits = r.integers(0, 2**32, size=100000, dtype=np.uint64).astype(np.uint32)
    else:
        bits = ALL16
    v = oracle.decode(bits, dtype)
    fin = np.isfinite(v)
    assert np.array_equal(oracle.encode(v[fin], dtype), bits[fin])
