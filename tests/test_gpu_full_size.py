"""GPU parity at the workloads' full sizes, every output element.

Each workload runs in the launch configuration the benchmark times (the
automatic tile, split and column split; stream-K and the fused q4 kernel
through their own entry points) and is compared element by element with the
oracle on the same seeded host arrays:

  * 4096^3 fp16 and bf16 operands N(0,1)/sqrt(K), fp16 and fp32 output;
  * 4096^3 small-integer operands, bit for bit (fp16 and fp32 output);
  * the fp32 ladder, n in {1024, 2048, 4096}, every rung;
  * the 2048-token prefill projections (q4_0 weights) through the two-pass
    route, the fused q4 kernel, the fp16 GEMM on the dequantised weight and
    the stream-K schedule, plus the q4_K / q6_K / padded q6_K two-pass route
    (the q4_K decode is parity unpinned by the pages: its layout is a reading
    from outside them, and only the oracle's own reading checks it);
  * the tall-skinny 65536 x 160 x {160, 32} bias+GELU products, whose
    second persistent step only runs at this size.

Floating-point results are judged by the normwise bound and by
|C_ij - T_ij| <= 1e-2 |alpha| U_ij + 1e-3 on every element.  The oracle's
products are computed once per session and shared between the routes that
must reproduce them.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, assert_close, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _ws_bytes(n):
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None


def _ws(M, N, K, dtype=torch.float16):
    return _ws_bytes(dge.gemm_workspace_size(M, N, K, dtype))


# ------------------------------------------------------------ oracle, cached

@functools.lru_cache(maxsize=None)
def _square(dtype):
    A, B = inputs.square4096(dtype)
    T, U = oracle.gemm(A, B, dtype)
    return A, B, T, U


@functools.lru_cache(maxsize=None)
def _square_int():
    r = np.random.Generator(np.random.PCG64(2042))
    A = inputs.to_bits(r.integers(-4, 5, (4096, 4096)).astype(float), "f16")
    B = inputs.to_bits(r.integers(-4, 5, (4096, 4096)).astype(float), "f16")
    T, _ = oracle.gemm(A, B, "f16", want_U=False)
    return A, B, T


@functools.lru_cache(maxsize=None)
def _prefill(shape):
    A, q, N, K = inputs.prefill_projection(shape)
    W16 = oracle.dequant_q4(q, N, K)
    T, U = oracle.gemm(A, W16, "f16", trans_b=True)
    return A, q, W16, T, U


# ------------------------------------------------------------ 4096^3

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("out", [torch.float16, torch.float32])
def test_square_4096_every_element(dtype, out):
    A, B, T, U = _square(dtype)
    C = dge.gemm(to_dev(A, dtype), to_dev(B, dtype), out_dtype=out,
                 workspace=_ws(4096, 4096, 4096, {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]))
    torch.cuda.synchronize()
    assert_close(C, T, U, what="%s -> %s" % (dtype, out))


@pytest.mark.parametrize("out", [torch.float32, torch.float16])
def test_square_4096_integer_bit_exact_every_element(out):
    A, B, T = _square_int()
    C = dge.gemm_f16(to_dev(A, "f16"), to_dev(B, "f16"), out_dtype=out,
                     workspace=_ws(4096, 4096, 4096))
    torch.cuda.synchronize()
    assert_bits(C, T, what=str(out))


@pytest.mark.parametrize("n", [1024, 2048, 4096])
def test_fp32_ladder_every_element(n):
    A, B = inputs.fp32_square(n)
    dA, dB = to_dev(A, "f32"), to_dev(B, "f32")
    T, U = oracle.gemm(A, B, "f32")
    for algo in ["naive", "lds_tiled", "mfma"]:
        C = dge.gemm_ex(dA, dB, out_dtype=torch.float32, algo=algo)
        torch.cuda.synchronize()
        assert_close(C, T, U, what="n=%d %s" % (n, algo))
        del C
    # with the workspace the library asks for (the schedule the benchmark
    # times: a K split at n = 1024)
    C = dge.gemm_ex(dA, dB, out_dtype=torch.float32, algo="mfma",
                    workspace=_ws(n, n, n, torch.float32))
    torch.cuda.synchronize()
    assert_close(C, T, U, what="n=%d mfma with workspace" % n)


# ------------------------------------------------------------ prefill, q4_0

@pytest.mark.parametrize("shape", ["up", "attn", "down"])
def test_prefill_two_pass_every_element(shape):
    A, q, W16, T, U = _prefill(shape)
    N, K = W16.shape
    w16 = torch.empty((N, K), dtype=torch.float16, device="cuda")
    C = dge.prefill_q4_f16(to_dev(A, "f16"), torch.from_numpy(q).cuda(), N, K, w16=w16,
                           workspace=_ws(2048, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(w16), W16), "dequantised weight, bit for bit"
    assert_close(C, T, U, what=shape)


@pytest.mark.parametrize("shape", ["up", "attn", "down"])
def test_prefill_fused_q4_every_element(shape):
    A, q, W16, T, U = _prefill(shape)
    N, K = W16.shape
    C = dge.gemm_q4_f16(to_dev(A, "f16"), torch.from_numpy(q).cuda(), N, K,
                        workspace=_ws(2048, N, K), algo="mfma_direct")
    torch.cuda.synchronize()
    assert_close(C, T, U, what=shape + " fused")


@pytest.mark.parametrize("shape", ["up", "attn", "down"])
def test_prefill_gemm_and_streamk_every_element(shape):
    # the fp16 GEMM on the dequantised weight (the bench's GEMM-only leg) and
    # the persistent stream-K schedule on the same operands
    A, q, W16, T, U = _prefill(shape)
    N, K = W16.shape
    dA, dW = to_dev(A, "f16"), to_dev(W16, "f16")
    C = dge.gemm_f16(dA, dW, trans_b=True, workspace=_ws(2048, N, K))
    torch.cuda.synchronize()
    assert_close(C, T, U, what=shape + " gemm_f16")
    ws = _ws_bytes(dge.gemm_workspace_size_streamk(2048, N, K))
    C = dge.gemm_ex(dA, dW, trans_b=True, workspace=ws, algo="streamk")
    torch.cuda.synchronize()
    assert_close(C, T, U, what=shape + " stream-K")


# ------------------------------------------------------------ prefill, K-quants

@pytest.mark.parametrize("qtype,shape", [(t, s) for t in ("q4_k", "q6_k")
                                          for s in ("up", "attn", "down")] + [("q6_k_224", "attn")])
def test_prefill_kquant_every_element(qtype, shape):
    A, q, N, K = inputs.kquant_projection(qtype, shape)
    W16 = oracle.dequant(qtype, q, N, K)
    w16 = torch.empty((N, K), dtype=torch.float16, device="cuda")
    C = dge.prefill_f16(qtype, to_dev(A, "f16"), torch.from_numpy(q).cuda(), N, K, w16=w16,
                        workspace=_ws(2048, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(w16), W16), "dequantised weight, bit for bit"
    T, U = oracle.gemm(A, W16, "f16", trans_b=True)
    assert_close(C, T, U, what="%s %s" % (qtype, shape))


# ------------------------------------------------------------ tall-skinny

@pytest.mark.parametrize("N", [160, 32])
def test_tall_skinny_bias_gelu_every_element(N):
    X, W, bias = inputs.tall_skinny(N)
    C = dge.gemm_f16(to_dev(X, "f16"), to_dev(W, "f16"), out_dtype=torch.float16,
                     epi="bias_gelu", bias=to_dev(bias, "f16"))
    torch.cuda.synchronize()
    T, U = oracle.gemm(X, W, "f16", epi="bias_gelu", bias=oracle.decode(bias, "f16"))
    assert_close(C, T, U, what="N=%d" % N)
