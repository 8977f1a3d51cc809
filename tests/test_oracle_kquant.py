"""Pins of the oracle's K-quant dequantisation (q6_K and q4_K super-blocks).

* Hand-derived blocks (tests/golden/kquant_blocks.txt): field offsets, the
  quarter / nibble / scale addressing, the 6-bit scale packing, and the
  float-then-half rounding of q4_K.
* Round trips through an independent packer written here from the layout
  (per element: where its bits go), decoded by the oracle and compared with
  numpy's own casts of the exact value (float16 for q6_K, float32 then
  float16 for q4_K).
* Every binary16 pattern of the q6_K scale d against numpy.
"""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kquant_blocks.txt")


def _golden():
    entries, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "name":
            cur = {"name": rest}
            entries.append(cur)
        elif key == "type":
            cur["type"] = rest
        elif key == "block":
            cur["block"] = np.array([int(x, 16) for x in rest.split()], dtype=np.uint8)
        elif key == "expect":
            vals = []
            for run in rest.split():
                n, _, v = run.partition("x")
                vals += [float(v)] * int(n)
            cur["expect"] = np.array(vals)
    return entries


def test_golden_blocks():
    entries = _golden()
    assert {e["type"] for e in entries} == {"q6_k", "q4_k"}
    for e in entries:
        got = oracle.dequant(e["type"], e["block"], 1, 256)[0].view(np.float16).astype(np.float64)
        assert got.shape == e["expect"].shape, e["name"]
        assert np.array_equal(got, e["expect"]), e["name"]


# ---- independent packers (element -> bits), written from the layout

def _pack_q6_k(d_bits, sc, codes):
    """d_bits: (S,) binary16 bits; sc: (S, 16) int8; codes: (S, 256) in 0..63."""
    S = len(d_bits)
    out = np.zeros((S, 210), dtype=np.uint8)
    for s in range(S):
        for e in range(256):
            h, tt, l = e // 128, (e % 128) // 32, e % 32
            low, high = int(codes[s, e]) & 15, int(codes[s, e]) >> 4
            qi = 64 * h + 32 * (tt & 1) + l
            out[s, qi] |= low if tt < 2 else low << 4
            out[s, 128 + 32 * h + l] |= high << (2 * tt)
        out[s, 192:208] = sc[s].astype(np.int8).view(np.uint8)
        out[s, 208] = d_bits[s] & 0xFF
        out[s, 209] = d_bits[s] >> 8
    return out.reshape(-1)


def _pack_q4_k(d_bits, dmin_bits, sc, m, codes):
    """sc, m: (S, 8) in 0..63; codes: (S, 256) in 0..15."""
    S = len(d_bits)
    out = np.zeros((S, 144), dtype=np.uint8)
    for s in range(S):
        out[s, 0], out[s, 1] = d_bits[s] & 0xFF, d_bits[s] >> 8
        out[s, 2], out[s, 3] = dmin_bits[s] & 0xFF, dmin_bits[s] >> 8
        k = out[s, 4:16]
        for j in range(4):
            k[j] |= sc[s, j]
            k[j + 4] |= m[s, j]
        for j in range(4, 8):
            k[j + 4] |= (sc[s, j] & 15) | ((m[s, j] & 15) << 4)
            k[j - 4] |= (sc[s, j] >> 4) << 6
            k[j] |= (m[s, j] >> 4) << 6
        for e in range(256):
            p, w = e // 64, e % 64
            byte = 16 + 32 * p + w % 32
            out[s, byte] |= codes[s, e] if w < 32 else codes[s, e] << 4
    return out.reshape(-1)


def _sub(e):
    # q4_K sub-block of weight e: pairs of 64 weights are sub-blocks 2p, 2p+1
    return 2 * (e // 64) + (e % 64 >= 32)


def test_q6_k_round_trip_matches_numpy():
    r = np.random.Generator(np.random.PCG64(7000))
    S = 24
    d = np.abs(r.normal(0, 0.01, S)).astype(np.float16)
    sc = r.integers(-128, 128, (S, 16))
    codes = r.integers(0, 64, (S, 256))
    q = _pack_q6_k(d.view(np.uint16), sc, codes)
    got = oracle.dequant("q6_k", q, S, 256)
    h, tt, l = np.arange(256) // 128, (np.arange(256) % 128) // 32, np.arange(256) % 32
    sidx = 8 * h + 2 * tt + l // 16
    exact = d.astype(np.float64)[:, None] * sc[:, sidx] * (codes - 32)
    assert np.array_equal(got, exact.astype(np.float16).view(np.uint16))


def test_q4_k_round_trip_matches_numpy():
    r = np.random.Generator(np.random.PCG64(7100))
    S = 24
    d = np.abs(r.normal(0, 0.05, S)).astype(np.float16)
    dmin = np.abs(r.normal(0, 0.05, S)).astype(np.float16)
    sc = r.integers(0, 64, (S, 8))
    m = r.integers(0, 64, (S, 8))
    codes = r.integers(0, 16, (S, 256))
    q = _pack_q4_k(d.view(np.uint16), dmin.view(np.uint16), sc, m, codes)
    got = oracle.dequant("q4_k", q, S, 256)
    j = np.array([_sub(e) for e in range(256)])
    t = d.astype(np.float64)[:, None] * sc[:, j] * codes
    u = dmin.astype(np.float64)[:, None] * m[:, j]
    want = (t - u).astype(np.float32).astype(np.float16)
    assert np.array_equal(got, want.view(np.uint16))


def test_q6_k_every_scale_pattern():
    # 65536 super-blocks, one per binary16 pattern of d; fixed codes and scales
    S = 65536
    d_bits = np.arange(S, dtype=np.uint32).astype(np.uint16)
    sc = np.tile(np.array([1, -1, 2, -2, 3, -3, 4, -4, 5, -5, 127, -128, 7, -7, 8, -8]), (S, 1))
    codes = np.tile(np.arange(256) % 64, (S, 1))
    one = _pack_q6_k(d_bits[:1], sc[:1], codes[:1]).reshape(1, 210)
    q = np.repeat(one, S, axis=0)
    q[:, 208] = d_bits & 0xFF
    q[:, 209] = d_bits >> 8
    got = oracle.dequant("q6_k", q.reshape(-1), S, 256).view(np.float16).astype(np.float64)
    h, tt, l = np.arange(256) // 128, (np.arange(256) % 128) // 32, np.arange(256) % 32
    sidx = 8 * h + 2 * tt + l // 16
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        want = (d[:, None] * sc[:, sidx] * (codes - 32)).astype(np.float16).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_q6_k_padded_stride_ignores_the_padding():
    # the same super-blocks at a 224-byte stride, 14 random bytes after each
    r = np.random.Generator(np.random.PCG64(7200))
    S = 12
    q = _pack_q6_k(np.abs(r.normal(0, 0.01, S)).astype(np.float16).view(np.uint16),
                   r.integers(-128, 128, (S, 16)), r.integers(0, 64, (S, 256)))
    padded = r.integers(0, 256, (S, 224), dtype=np.uint8)
    padded[:, :210] = q.reshape(S, 210)
    want = oracle.dequant("q6_k", q, 3, 4 * 256)
    assert np.array_equal(oracle.dequant("q6_k_224", padded.reshape(-1), 3, 4 * 256), want)
    # the padding really is skipped: shifting it into a block changes the result
    assert not np.array_equal(oracle.dequant("q6_k", padded.reshape(-1)[: S * 210], 3, 4 * 256),
                              want)


def test_shapes_rejected():
    import pytest
    with pytest.raises(ValueError):
        oracle.dequant("q6_k", np.zeros(210, np.uint8), 1, 128)
    with pytest.raises(ValueError):
        oracle.dequant("q4_k", np.zeros(100, np.uint8), 1, 256)
