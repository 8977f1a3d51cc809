"""GPU parity of the decode-shaped kernel (1 <= M <= 64 input rows against an
N x K weight) against the oracle: integer-valued inputs bit for bit (every
partial sum is an exact fp32 integer, and the 8 K-slice partials are summed
in a fixed order), random inputs and the epilogues by the tolerance, and the
4096 x 4096 decode workload in full.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _ints(shape, dtype, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return inputs.to_bits(r.integers(-4, 5, shape).astype(float), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 512, 256), (5, 100, 40), (16, 64, 8), (17, 300, 1000),
                                   (33, 16, 4096), (64, 1040, 520),
                                   # whole-row weight batches: ragged N (clamped rows), two
                                   # batches per wave, a batch plus a ragged end
                                   (8, 100, 4096), (16, 256, 8192), (2, 48, 4160), (1, 80, 4096)])
def test_decode_integer_exact_and_deterministic(M, N, K, dtype):
    X, W = _ints((M, K), dtype, 6000 + M), _ints((N, K), dtype, 6100 + N)
    T, _ = oracle.gemm(X, W, dtype, trans_b=True, want_U=False)
    outs = []
    for _ in range(2):
        C = dge.gemm_ex(to_dev(X, dtype), to_dev(W, dtype), trans_b=True,
                        out_dtype=torch.float32, algo="decode")
        torch.cuda.synchronize()
        assert_bits(C, T, what="%dx%dx%d %s" % (M, N, K, dtype))
        outs.append(C.cpu())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("out", [torch.float16, torch.float32, torch.bfloat16])
def test_decode_epilogues_alpha_beta(out):
    M, N, K = 24, 200, 512
    r = np.random.Generator(np.random.PCG64(6200))
    X = inputs.to_bits(r.normal(0, 1, (M, K)), "f16")
    W = inputs.to_bits(r.normal(0, 1 / np.sqrt(K), (N, K)), "f16")
    bias_bits = inputs.to_bits(r.normal(0, 0.1, N), "f16")
    bias = oracle.decode(bias_bits, "f16")
    c_old = torch.from_numpy(r.normal(0, 1, (M, N))).to(out).cuda()
    C = c_old.clone()
    dge.gemm_ex(to_dev(X, "f16"), to_dev(W, "f16"), C, trans_b=True, alpha=0.5, beta=-1.0,
                epi="bias_gelu", bias=to_dev(bias_bits, "f16"), algo="decode")
    torch.cuda.synchronize()
    cold = c_old.double().cpu().numpy()
    T, U = oracle.gemm(X, W, "f16", trans_b=True, alpha=0.5, beta=-1.0, C_old=cold,
                       epi="bias_gelu", bias=bias)
    assert_close(C, T, U, alpha=0.5)


@pytest.mark.parametrize("M", inputs.DECODE_ROWS)
def test_decode_workload_4096_full(M):
    # the automatic choice takes the decode kernel for this shape
    X, W = inputs.decode_shape(M)
    C = dge.gemm_f16(to_dev(X, "f16"), to_dev(W, "f16"), trans_b=True, out_dtype=torch.float16)
    torch.cuda.synchronize()
    T, U = oracle.gemm(X, W, "f16", trans_b=True)
    assert_close(C, T, U, what="M=%d" % M)


def test_decode_misaligned_falls_back():
    # a weight view at an odd element offset is not 16-byte aligned: the
    # general kernel takes it, with the same result
    M, N, K = 3, 96, 64
    X, Wb = _ints((M, K), "f16", 6300), _ints((N, K + 1), "f16", 6301)
    W = Wb[:, 1:]
    T, _ = oracle.gemm(X, np.ascontiguousarray(W), "f16", trans_b=True, want_U=False)
    dW = to_dev(Wb, "f16")[:, 1:]
    C = dge.gemm_ex(to_dev(X, "f16"), dW, trans_b=True, out_dtype=torch.float32, algo="decode")
    torch.cuda.synchronize()
    assert_bits(C, T)


def _split_ws(M, N, K, dtype):
    n = dge.gemm_workspace_size(M, N, K, {"f16": torch.float16, "bf16": torch.bfloat16}[dtype])
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(33, 64, 4096), (32, 4096, 4096), (48, 1088, 11008),
                                   (64, 4096, 4096), (64, 128, 8192), (40, 192, 256),
                                   (17, 256, 4096), (24, 4096, 1056)])
def test_decode_split_integer_exact_and_deterministic(M, N, K, dtype):
    # with a workspace, 17 <= M <= 64 splits K over workgroups of 64 weight
    # rows (uneven slices at K = 11008; at K = 1056 every wave has a single
    # k-block, below a whole 4-block span); the fp32 partials are summed in slice
    # order, so integer inputs give the oracle's bits on every run
    X, W = _ints((M, K), dtype, 6400 + M), _ints((N, K), dtype, 6500 + N)
    T, _ = oracle.gemm(X, W, dtype, trans_b=True, want_U=False)
    ws = _split_ws(M, N, K, dtype)
    outs = []
    for _ in range(2):
        C = dge.gemm_ex(to_dev(X, dtype), to_dev(W, dtype), trans_b=True,
                        out_dtype=torch.float32, algo="decode", workspace=ws)
        torch.cuda.synchronize()
        assert_bits(C, T, what="%dx%dx%d %s" % (M, N, K, dtype))
        outs.append(C.cpu())
    assert torch.equal(outs[0], outs[1])


def test_decode_split_any_workspace_contents():
    # the split schedule overwrites its whole partial area before reading
    # it: a workspace full of arbitrary bits, or just used by a split-K GEMM
    # and by a decode of another shape, gives the same bits
    M, N, K = 64, 1024, 4096
    X, W = _ints((M, K), "f16", 6700), _ints((N, K), "f16", 6701)
    T, _ = oracle.gemm(X, W, "f16", trans_b=True, want_U=False)
    nbytes = max(dge.gemm_workspace_size(M, N, K, torch.float16),
                 dge.gemm_workspace_size_splits(256, 512, 4), 1 << 20)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(6702)
    ws.view(torch.int32).copy_(torch.randint(-2**31, 2**31 - 1, (ws.numel(),), generator=g,
                                             dtype=torch.int32))
    dX, dW = to_dev(X, "f16"), to_dev(W, "f16")
    for step in range(3):
        C = dge.gemm_ex(dX, dW, trans_b=True, out_dtype=torch.float32, algo="decode",
                        workspace=ws)
        torch.cuda.synchronize()
        assert_bits(C, T, what="step %d" % step)
        # other users of the same workspace between the calls
        A2 = torch.ones((256, 4096), dtype=torch.float16, device="cuda")
        B2 = torch.ones((4096, 512), dtype=torch.float16, device="cuda")
        dge.gemm_ex(A2, B2, workspace=ws, algo="mfma", splits=4)
        dge.gemm_ex(dX[:40], dW[:192], trans_b=True, algo="decode", workspace=ws)
        torch.cuda.synchronize()


def test_decode_split_epilogue():
    M, N, K = 40, 512, 4096
    r = np.random.Generator(np.random.PCG64(6600))
    X = inputs.to_bits(r.normal(0, 1, (M, K)), "f16")
    W = inputs.to_bits(r.normal(0, 1 / np.sqrt(K), (N, K)), "f16")
    bias_bits = inputs.to_bits(r.normal(0, 0.1, N), "f16")
    cold_bits = inputs.to_bits(r.normal(0, 1, (M, N)), "f16")
    C = to_dev(cold_bits, "f16")
    dge.gemm_f16(to_dev(X, "f16"), to_dev(W, "f16"), C, trans_b=True, alpha=0.5, beta=-1.0,
                 epi="bias_gelu", bias=to_dev(bias_bits, "f16"), workspace=_split_ws(M, N, K, "f16"))
    torch.cuda.synchronize()
    T, U = oracle.gemm(X, W, "f16", trans_b=True, alpha=0.5, beta=-1.0,
                       C_old=oracle.decode(cold_bits, "f16"), epi="bias_gelu",
                       bias=oracle.decode(bias_bits, "f16"))
    assert_close(C, T, U, alpha=0.5)


@pytest.mark.parametrize("M", inputs.DECODE_ROWS)
def test_decode_workload_4096_with_workspace(M):
    # the launch configuration the benchmark times (workspace from
    # gemm_workspace_size: the split schedule for M = 64)
    X, W = inputs.decode_shape(M)
    C = dge.gemm_f16(to_dev(X, "f16"), to_dev(W, "f16"), trans_b=True, out_dtype=torch.float16,
                     workspace=_split_ws(M, 4096, 4096, "f16"))
    torch.cuda.synchronize()
    T, U = oracle.gemm(X, W, "f16", trans_b=True)
    assert_close(C, T, U, what="M=%d" % M)
