"""GPU parity of the q4 dequant (bit for bit: every scale pattern, every
code, the full prefill weights, ragged, strided and unaligned layouts), the
prefill page's tail shape, and the column-split schedule.  The full-size
products are compared element by element in test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, assert_close, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _ws(M, N, K, dtype=torch.float16):
    n = dge.gemm_workspace_size(M, N, K, dtype)
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None


def test_dequant_every_scale_times_every_code():
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    codes = np.empty((65536, 1, 32), dtype=np.uint8)
    codes[:, 0, :16] = np.arange(16)
    codes[:, 0, 16:] = np.arange(15, -1, -1)
    q = inputs.pack_q4(scales[:, None], codes)
    want = oracle.dequant_q4(q, 65536, 32)
    got = bits_of(dge.dequant_q4_f16(torch.from_numpy(q).cuda(), 65536, 32))
    d = scales.view(np.float16).astype(np.float64)
    fin = np.isfinite(d)
    assert np.array_equal(got[fin], want[fin])
    # non-finite scales: same class (NaN / signed inf) per element
    g = got[~fin].view(np.float16).astype(np.float64)
    w = want[~fin].view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    assert np.array_equal(g[~np.isnan(g)], w[~np.isnan(w)])


def test_dequant_256_wide_rows_every_scale_times_every_code():
    # rows of 256 weights (eight blocks) take the grouped path: every scale
    # pattern once, each block holding codes 0..15 and 15..0
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(8192, 8)
    codes = np.empty((8192, 8, 32), dtype=np.uint8)
    codes[:, :, :16] = np.arange(16)
    codes[:, :, 16:] = np.arange(15, -1, -1)
    q = inputs.pack_q4(scales, codes)
    want = oracle.dequant_q4(q, 8192, 256)
    got = bits_of(dge.dequant_q4_f16(torch.from_numpy(q).cuda(), 8192, 256))
    torch.cuda.synchronize()
    g, w = got.view(np.float16), want.view(np.float16)
    # bit for bit, any NaN matching any NaN (non-finite scales)
    assert np.all((got == want) | (np.isnan(g) & np.isnan(w)))


@pytest.mark.parametrize("rows,cols,ldo,qoff", [(37, 512, 520, 0), (5, 768, 771, 0),
                                                (9, 256, 256, 2), (300, 1024, 1024, 16)])
def test_dequant_grouped_path_strided_and_unaligned(rows, cols, ldo, qoff):
    q = inputs.q4_weights(rows, cols, 4, 93 + rows)
    buf = torch.zeros(q.size + qoff, dtype=torch.uint8, device="cuda")
    buf[qoff:] = torch.from_numpy(q).cuda()
    out = torch.full((rows, ldo), float("nan"), dtype=torch.float16, device="cuda")
    dge.dequant_q4_f16(buf[qoff:], rows, cols, out=out[:, :cols])
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out[:, :cols]), oracle.dequant_q4(q, rows, cols))
    assert torch.all(torch.isnan(out[:, cols:]))


@pytest.mark.parametrize("shape", ["up", "attn", "down"])
def test_dequant_full_size_bit_exact(shape):
    N, K = inputs.PREFILL_SHAPES[shape]
    q = inputs.q4_weights(N, K, 4, {"up": 0, "attn": 1, "down": 2}[shape])
    got = dge.dequant_q4_f16(torch.from_numpy(q).cuda(), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(got), oracle.dequant_q4(q, N, K))


def test_dequant_ragged_rows_and_padded_output():
    rows, cols, ldo = 37, 96, 100
    q = inputs.q4_weights(rows, cols, 91)
    out = torch.full((rows, ldo), float("nan"), dtype=torch.float16, device="cuda")
    dge.dequant_q4_f16(torch.from_numpy(q).cuda(), rows, cols, out=out[:, :cols])
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out[:, :cols]), oracle.dequant_q4(q, rows, cols))
    assert torch.all(torch.isnan(out[:, cols:]))


def test_dequant_rejects_ragged_cols():
    q = torch.zeros(18 * 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(dge.GemmError):
        dge.dequant_q4_f16(q, 4, 16)


def test_prefill_tail_shape_unit_scales_exact():
    # the prefill page's tail shape (od = 70, nt = 33, id = 256); d = 1 makes
    # W16 the integers q - 8, so the product is exact
    M, N, K = 33, 70, 256
    r = np.random.Generator(np.random.PCG64(5000))
    codes = r.integers(0, 16, (N, K // 32, 32))
    q = inputs.pack_q4(np.full((N, K // 32), 0x3C00, dtype=np.uint16), codes)
    A = inputs.to_bits(r.integers(-4, 5, (M, K)).astype(float), "f16")
    C = dge.prefill_q4_f16(to_dev(A, "f16"), torch.from_numpy(q).cuda(), N, K,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    T, _, _ = oracle.prefill(A, q, N, K, want_U=False)
    assert_bits(C, T)


@pytest.mark.parametrize("trans_b", [False, True])
def test_column_split_schedule_integer_exact(trans_b, monkeypatch):
    # 2048 x 11008: 344 tiles of 256 x 256 for 256 CUs, so the automatic
    # schedule runs 8192 columns as one full round and the other 2816 on
    # their own; small-integer inputs make every partial sum exact, so both
    # parts (and the same problem without the column split) give the
    # oracle's bits, bias included
    M, N, K = 2048, 11008, 512
    r = np.random.Generator(np.random.PCG64(9100 + trans_b))
    A = inputs.to_bits(r.integers(-4, 5, (M, K)).astype(float), "f16")
    B = inputs.to_bits(r.integers(-4, 5, (N, K) if trans_b else (K, N)).astype(float), "f16")
    bias_bits = inputs.to_bits(r.integers(-8, 9, N).astype(float), "f16")
    bias = oracle.decode(bias_bits, "f16")
    T, _ = oracle.gemm(A, B, "f16", trans_b=trans_b, epi="bias", bias=bias, want_U=False)
    n = dge.gemm_workspace_size(M, N, K, torch.float16)
    ws = torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda")
    for colsplit in ("1", "0"):
        monkeypatch.setenv("GEMM_COLSPLIT", colsplit)
        C = dge.gemm_f16(to_dev(A, "f16"), to_dev(B, "f16"), trans_b=trans_b,
                         out_dtype=torch.float32, epi="bias", bias=to_dev(bias_bits, "f16"),
                         workspace=ws)
        torch.cuda.synchronize()
        assert_bits(C, T, what="colsplit=%s" % colsplit)
