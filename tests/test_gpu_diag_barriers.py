"""The pipelined direct-to-LDS kernels against their diagnostic build.

libdge_gemm_diag.so is the same library compiled with
GEMM_DIAG_EXTRA_BARRIERS: after every group of direct loads, fragment reads,
q4 decode writes and epilogue staging writes each wave waits for its memory
operations and meets every other wave at a barrier, so nothing overlaps.  On
small-integer inputs (every partial sum exact in fp32) both builds must give
the oracle's bits: a missing wait or barrier in the overlapped schedule (a
wave's loads landing in a buffer another wave still reads) would make the
normal build differ.  Covered: every direct tile in both B layouts at one,
two, three and many stages, split-K slices, the fused q4 kernel and the
stream-K schedule.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, bits_of, to_dev

pytestmark = pytest.mark.gpu

TILES = ["256x256w8", "256x128w8", "256x256", "256x128", "128x128", "128x64"]


def _ints(shape, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return inputs.to_bits(r.integers(-4, 5, shape).astype(float), "f16")


def _both(fn):
    a = fn()
    torch.cuda.synchronize()
    with dge.diag_library():
        b = fn()
        torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("K", [64, 128, 192, 1024])
def test_direct_tiles_match_the_diagnostic_build(K, trans_b):
    M, N = 512, 512
    A = _ints((M, K), 9700 + K)
    B = _ints((N, K) if trans_b else (K, N), 9701 + K)
    T, _ = oracle.gemm(A, B, "f16", trans_b=trans_b, want_U=False)
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    for tile in TILES:
        if tile == "128x64" and not trans_b:
            continue  # the register-staged kernel runs it
        a, b = _both(lambda: dge.gemm_ex(dA, dB, trans_b=trans_b, out_dtype=torch.float32,
                                         algo="mfma_direct", tile=tile, splits=1,
                                         epi="bias", bias=torch.ones(N, dtype=torch.float16,
                                                                     device="cuda")))
        assert np.array_equal(bits_of(a), bits_of(b)), tile
        assert_bits(a, T + 1.0, what=tile)


def test_split_k_and_fused_q4_match_the_diagnostic_build():
    M, N, K = 512, 512, 2048
    A = _ints((M, K), 9800)
    B = _ints((N, K), 9801)
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    ws = torch.empty(dge.gemm_workspace_size_splits(M, N, 3) // 4, dtype=torch.float32,
                     device="cuda")
    for tile in ("256x256w8", "256x128w8"):
        a, b = _both(lambda: dge.gemm_ex(dA, dB, trans_b=True, out_dtype=torch.float32,
                                         workspace=ws, algo="mfma_direct", tile=tile, splits=3))
        assert np.array_equal(bits_of(a), bits_of(b)), tile
    # fused q4 with unit scales: W = codes - 8, integer products
    r = np.random.Generator(np.random.PCG64(9802))
    q = inputs.pack_q4(np.full((N, K // 32), 0x3C00, dtype=np.uint16),
                       r.integers(0, 16, (N, K // 32, 32)))
    dq = torch.from_numpy(q).cuda()
    T, _, _ = oracle.prefill(A, q, N, K, want_U=False)
    for tile in ("256x256w8", "256x128w8"):
        a, b = _both(lambda: dge.gemm_q4_f16(dA, dq, N, K, out_dtype=torch.float32,
                                             algo="mfma_direct", tile=tile))
        assert np.array_equal(bits_of(a), bits_of(b)), tile
        assert_bits(a, T, what="q4 " + tile)


def test_streamk_matches_the_diagnostic_build():
    M, N, K = 1024, 1280, 2048
    A = _ints((M, K), 9900)
    B = _ints((N, K), 9901)
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    ws = torch.empty(dge.gemm_workspace_size_streamk(M, N, K) // 4, dtype=torch.float32,
                     device="cuda")
    a, b = _both(lambda: dge.gemm_ex(dA, dB, trans_b=True, out_dtype=torch.float32,
                                     workspace=ws, algo="streamk"))
    assert np.array_equal(bits_of(a), bits_of(b))
