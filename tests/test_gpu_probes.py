"""The measurement probes (include/gemm_probe.h) compute what they claim.

* gemm_probe_clock gives the same bits as the GEMM it instruments and
  sensible clock records (shader cycles per real-time tick in a plausible
  engine-clock range, end after start).
* gemm_probe_mfma does the MFMA work it is priced at: with small-integer
  operands every lane's sum is exact in fp32 and equals the same sum of
  products computed with integers on the host (the lane -> row / column map
  of a 16x16x32 block with swapped operands).
* gemm_probe_phases gives the same bits as the split decode and tall-skinny
  schedules it instruments and ordered phase records, one set per workgroup.
* the streaming probes read / copy every byte.
"""
import numpy as np
import pytest
import torch

import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu


def test_probe_phases_split_decode():
    M, N, K = 64, 4096, 4096
    X, W = inputs.decode_shape(M)
    dX, dW = to_dev(X, "f16"), to_dev(W, "f16")
    ws = torch.empty(dge.gemm_workspace_size(M, N, K, torch.float16) // 4, dtype=torch.float32,
                     device="cuda")
    C0 = dge.gemm_f16(dX, dW, trans_b=True, workspace=ws)
    C1 = torch.empty_like(C0)
    rec = torch.zeros(4 * 300, dtype=torch.int64, device="cuda")
    dge.probe_phases(dX, dW, C1, rec, trans_b=True, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C0), bits_of(C1))
    r = rec.view(-1, 4).cpu().numpy()
    nwg = N // 64 * 4  # 4 K slices of 64 weight rows
    assert np.all(r[nwg:] == 0)
    r = r[:nwg].astype(np.float64)
    assert np.all(np.diff(r, axis=1) >= 0), "phases out of order"
    span_us = (r[:, 3].max() - r[:, 0].min()) / 100.0
    assert 0.5 < span_us < 1000.0, span_us
    # a grid larger than the records, and a schedule without phase records
    with pytest.raises(dge.GemmError) as e:
        dge.probe_phases(dX, dW, C1, rec[:4 * (nwg - 1)], trans_b=True, workspace=ws)
    assert e.value.status == 2
    with pytest.raises(dge.GemmError) as e:
        dge.probe_phases(dX, dW, C1, rec, trans_b=True)  # no workspace: one-pass kernel
    assert e.value.status == 2


@pytest.mark.parametrize("N", [160, 32])
def test_probe_phases_tall_skinny(N):
    X, W, bias = inputs.tall_skinny(N)
    dX, dW, db = to_dev(X, "f16"), to_dev(W, "f16"), to_dev(bias, "f16")
    C0 = dge.gemm_f16(dX, dW, epi="bias_gelu", bias=db)
    C1 = torch.empty_like(C0)
    rec = torch.zeros(4 * 300, dtype=torch.int64, device="cuda")
    dge.probe_phases(dX, dW, C1, rec, epi="bias_gelu", bias=db)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C0), bits_of(C1))
    r = rec.view(-1, 4).cpu().numpy()
    nwg = int((r[:, 0] != 0).sum())
    assert 1 <= nwg <= 256 and np.all(r[nwg:] == 0)
    r = r[:nwg].astype(np.float64)
    assert np.all(np.diff(r, axis=1) >= 0), "phases out of order"
    with pytest.raises(dge.GemmError) as e:
        dge.probe_phases(dX, dW, C1, rec[:4 * (nwg - 1)], epi="bias_gelu", bias=db)
    assert e.value.status == 2


def test_probe_clock_same_bits_and_sane_clock():
    A, B = inputs.square4096("f16")
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    C0 = dge.gemm_f16(dA, dB)
    C1 = torch.empty_like(C0)
    clk = torch.zeros(4 * 512, dtype=torch.int64, device="cuda")
    dge.probe_clock(dA, dB, C1, clk)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C0), bits_of(C1))
    c = clk.view(-1, 4).cpu().numpy().astype(np.float64)[:256]
    assert np.all(c[:, 2] > c[:, 0]) and np.all(c[:, 3] > c[:, 1])
    mhz = (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * 100.0
    assert 300.0 < np.median(mhz) < 3000.0, np.median(mhz)
    assert np.all(clk.view(-1, 4)[256:].cpu().numpy() == 0)  # one record per workgroup
    # a grid larger than the records is refused before anything runs
    with pytest.raises(dge.GemmError) as e:
        dge.probe_clock(dA, dB, C1, clk[:4 * 255])
    assert e.value.status == 2


@pytest.mark.parametrize("k_blocks", [2, 6])
def test_probe_mfma_exact_sums(k_blocks):
    r = np.random.Generator(np.random.PCG64(9900))
    a = r.integers(-4, 5, (4096, 64)).astype(np.int64)
    bt = r.integers(-4, 5, (4096, 64)).astype(np.int64)  # rows = output columns
    dA = to_dev(inputs.to_bits(a.astype(float), "f16"), "f16")
    dB = to_dev(inputs.to_bits(bt.astype(float), "f16"), "f16")
    out = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    dge.probe_mfma(dA, dB, k_blocks, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256, 8, 64)
    # k-blocks alternate between k 0..31 and 32..63; every partial product
    # sum is an integer far below 2^53, exact in binary64 matrix products
    reps = ((k_blocks + 1) // 2, k_blocks // 2)
    af, bf = a.astype(np.float64), bt.astype(np.float64)
    D = reps[0] * (af[:, :32] @ bf[:, :32].T) + reps[1] * (af[:, 32:] @ bf[:, 32:].T)
    lane = np.arange(64)
    want = np.zeros((256, 8, 64), dtype=np.int64)
    for w in range(256):
        tm, tn = w // 16, w % 16
        for wave in range(8):
            r0 = tm * 256 + (wave // 4) * 128
            c0 = tn * 256 + (wave % 4) * 64
            rows = r0 + 16 * np.arange(8)[:, None] + lane % 16                      # (8, 64)
            cols = (c0 + 16 * np.arange(4)[:, None, None] + 4 * (lane // 16)
                    + np.arange(4)[None, :, None])                                  # (4, 4, 64)
            want[w, wave] = D[rows[:, None, None, :], cols[None, :, :, :]].sum(axis=(0, 1, 2))
    assert np.array_equal(got.astype(np.int64), want)


def test_probe_stream_read_and_copy():
    n = (64 << 20) + 4096
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    words = src.cpu().numpy().view(np.uint32)
    for grid in (1000, 4096):
        out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        dge.probe_read(src, out, grid)
        dst = torch.zeros_like(src)
        dge.probe_copy(src, dst, grid)
        torch.cuda.synchronize()
        assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == \
            np.bitwise_xor.reduce(words)
        assert torch.equal(src, dst)
