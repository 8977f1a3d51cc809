"""gemm_ex_noalloc: gemm_ex with the library's static per-device scratch in
place of a caller workspace (for callers that cannot allocate).

Each case runs twice in a row on the same stream, the second time with a
smaller problem, so the second call meets the first call's leftovers in the
shared scratch; both must equal gemm_ex with a caller workspace of the same
size (the same schedule, so the same bits) and the oracle (bit for bit on
small-integer inputs, within the tolerance on random ones).
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, assert_close, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _operands(M, N, K, trans_b, integer, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    if integer:
        a = r.integers(-4, 5, (M, K)).astype(float)
        b = r.integers(-4, 5, (N, K) if trans_b else (K, N)).astype(float)
    else:
        a = r.normal(0, 1, (M, K)) / np.sqrt(K)
        b = r.normal(0, 1, (N, K) if trans_b else (K, N)) / np.sqrt(K)
    return inputs.to_bits(a, "f16"), inputs.to_bits(b, "f16")


def _with_workspace(dA, dB, trans_b, out, **kw):
    ws = torch.empty(dge.NOALLOC_SCRATCH_BYTES // 4, dtype=torch.float32, device="cuda")
    C = dge.gemm_ex(dA, dB, trans_b=trans_b, out_dtype=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    return C


# (M, N, K) of the first and the second, smaller, call; tuning
CASES = [
    # automatic schedule: both shapes split K (8 and 1 MiB of partials)
    ((512, 512, 8192), (256, 256, 4096), dict()),
    # explicit splits, the second leaving most of the first's partials behind
    ((1024, 512, 4096), (256, 384, 2048), dict(algo="mfma_direct", tile="256x128w8", splits=4)),
    # stream-K: partial tiles and arrival counters in the scratch
    # (256 x 256 x 2048: 256 (tile, stage) iterations on 256 workgroups, every
    # tile split into 32 pieces; 16 MiB of partial tiles)
    ((256, 256, 2048), (128, 192, 1024), dict(algo="streamk", tile="128x64")),
]


@pytest.mark.parametrize("first,second,kw,trans_b",
                         [c + (t,) for c in CASES for t in (True, False)
                          if t or c[2].get("tile") != "128x64"])  # 128 x 64: N x K B only
def test_noalloc_matches_gemm_ex_twice(first, second, kw, trans_b):
    for integer in (True, False):
        for (M, N, K), seed in ((first, 10), (second, 20)):
            A, B = _operands(M, N, K, trans_b, integer, seed + integer)
            dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
            out = torch.float32 if integer else torch.float16
            C = dge.gemm_ex_noalloc(dA, dB, trans_b=trans_b, out_dtype=out, **kw)
            torch.cuda.synchronize()
            ref = _with_workspace(dA, dB, trans_b, out, **kw)
            assert np.array_equal(bits_of(C), bits_of(ref)), (M, N, K, integer)
            T, U = oracle.gemm(A, B, "f16", trans_b=trans_b, want_U=not integer)
            if integer:
                assert_bits(C, T, what="%s %s" % ((M, N, K), kw))
            else:
                assert_close(C, T, U, what="%s %s" % ((M, N, K), kw))


def test_noalloc_epilogue_beta_and_bias():
    M, N, K = 512, 384, 8192
    A, B = _operands(M, N, K, False, False, 30)
    r = np.random.Generator(np.random.PCG64(31))
    bias_bits = inputs.to_bits(r.normal(0, 0.1, N), "f16")
    cold_bits = inputs.to_bits(r.normal(0, 1, (M, N)), "f16")
    dA, dB, db = to_dev(A, "f16"), to_dev(B, "f16"), to_dev(bias_bits, "f16")
    C = to_dev(cold_bits, "f16")
    dge.gemm_ex_noalloc(dA, dB, C, alpha=0.5, beta=-1.0, epi="bias_gelu", bias=db)
    ws = torch.empty(dge.NOALLOC_SCRATCH_BYTES // 4, dtype=torch.float32, device="cuda")
    ref = to_dev(cold_bits, "f16")
    dge.gemm_ex(dA, dB, ref, alpha=0.5, beta=-1.0, epi="bias_gelu", bias=db, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C), bits_of(ref))
    T, U = oracle.gemm(A, B, "f16", alpha=0.5, beta=-1.0, C_old=oracle.decode(cold_bits, "f16"),
                       epi="bias_gelu", bias=oracle.decode(bias_bits, "f16"))
    assert_close(C, T, U, alpha=0.5)


def test_noalloc_rejects_a_split_beyond_the_scratch():
    # 4 slices of a 2048 x 2048 fp32 partial need 64 MiB > 32 MiB
    M = N = 2048
    K = 4096
    dA = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    dB = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(dge.GemmError) as e:
        dge.gemm_ex_noalloc(dA, dB, C, algo="mfma_direct", splits=4)
    assert e.value.status == 6  # GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)  # nothing was enqueued
    # the automatic schedule of the same shape picks a split that fits
    dge.gemm_ex_noalloc(dA, dB, C)
    torch.cuda.synchronize()
    assert torch.all(C == 0.0)
