"""GPU parity of the fused q4-dequant GEMM (gemm_q4_f16) against the oracle.

The fused kernel decodes the q4 blocks inside the GEMM's B-tile producer, so
its decoding is checked through products that are exact: with A = I (one
1 per row), C = W^T holds every decoded weight once, in fp32, and must
equal the oracle's dequantisation exactly (as values: a zero weight's sign
is lost in the sum); with unit scales and
small-integer A every partial sum is an exact fp32 integer.  Random inputs
are judged by the tolerance (the prefill shapes, every element, in
test_gpu_full_size.py).
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_engineering_amd.binding as dge
from dense_gemm_engineering_amd import inputs
from gpu_util import assert_bits, assert_close, bits_of, to_dev

pytestmark = pytest.mark.gpu

FUSED_TILES = ["256x256w8", "256x128w8", "256x256", "256x128", "128x128", "128x64"]


def _q(q):
    return torch.from_numpy(np.ascontiguousarray(q)).cuda()


def _identity(n):
    return inputs.to_bits(np.eye(n), "f16")


def _unit_scale_q4(N, K, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    codes = r.integers(0, 16, (N, K // 32, 32))
    return inputs.pack_q4(np.full((N, K // 32), 0x3C00, dtype=np.uint16), codes)


def test_fused_decode_every_scale_times_every_code():
    # 65536 blocks, one per binary16 scale pattern, codes 0..15 and 15..0;
    # K = 256 (8 blocks per weight row), so a row holds 8 consecutive
    # patterns.  Rows holding a non-finite weight (a non-finite scale, or a
    # product that overflows binary16) are left out: 0 * inf in the other
    # terms of the product would make the whole row NaN.  The standalone
    # dequant test covers those values bit for bit.
    K = 256
    N = 65536 // (K // 32)
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(N, K // 32)
    codes = np.empty((N, K // 32, 32), dtype=np.uint8)
    codes[:, :, :16] = np.arange(16)
    codes[:, :, 16:] = np.arange(15, -1, -1)
    q = inputs.pack_q4(scales, codes)
    want = oracle.dequant_q4(q, N, K)  # N x K binary16 bits
    finite_rows = np.all(np.isfinite(want.view(np.float16)), axis=1)
    assert finite_rows.sum() > 0.85 * N
    A = to_dev(_identity(K), "f16")
    for tile in FUSED_TILES:
        C = dge.gemm_q4_f16(A, _q(q), N, K, out_dtype=torch.float32, algo="mfma_direct",
                            tile=tile)
        torch.cuda.synchronize()
        got = C.cpu().numpy().T  # N x K fp32: W[n][k]
        exp = want.view(np.float16).astype(np.float32)
        # exact equality of values; the sign of a zero weight does not survive
        # the product (the fp32 sum starts at +0, and +0 + -0 = +0)
        bad = got[finite_rows] != exp[finite_rows]
        assert not bad.any(), "tile %s: %d decoded weights differ" % (tile, int(bad.sum()))


@pytest.mark.parametrize("tile", FUSED_TILES)
def test_fused_unit_scales_integer_exact(tile):
    M, N, K = 512, 768, 1024
    q = _unit_scale_q4(N, K, 5100)
    r = np.random.Generator(np.random.PCG64(5101))
    A = inputs.to_bits(r.integers(-4, 5, (M, K)).astype(float), "f16")
    C = dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, out_dtype=torch.float32,
                        algo="mfma_direct", tile=tile)
    torch.cuda.synchronize()
    T, _, _ = oracle.prefill(A, q, N, K, want_U=False)
    assert_bits(C, T, what=tile)


@pytest.mark.parametrize("tile", ["256x256w8", "256x128w8"])
@pytest.mark.parametrize("splits", [2, 3])
def test_fused_split_k_exact_and_deterministic(splits, tile):
    M, N, K = 256, 512, 2048
    q = _unit_scale_q4(N, K, 5200)
    r = np.random.Generator(np.random.PCG64(5201))
    A = inputs.to_bits(r.integers(-4, 5, (M, K)).astype(float), "f16")
    ws = torch.empty(dge.gemm_workspace_size_splits(M, N, splits) // 4, dtype=torch.float32,
                     device="cuda")
    T, _, _ = oracle.prefill(A, q, N, K, want_U=False)
    outs = []
    for _ in range(2):
        C = dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, out_dtype=torch.float32, workspace=ws,
                            algo="mfma_direct", tile=tile, splits=splits)
        torch.cuda.synchronize()
        assert_bits(C, T, what="%s splits=%d" % (tile, splits))
        outs.append(C.cpu())
    assert torch.equal(outs[0], outs[1])


def test_fused_bias_gelu_epilogue():
    M, N, K = 256, 512, 512
    r = np.random.Generator(np.random.PCG64(5300))
    A = inputs.to_bits(r.normal(0, 1, (M, K)), "f16")
    q = inputs.q4_weights(N, K, 53)
    bias_bits = inputs.to_bits(r.normal(0, 0.1, N), "f16")
    bias = oracle.decode(bias_bits, "f16")
    C = dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, epi="bias_gelu",
                        bias=to_dev(bias_bits, "f16"), algo="mfma_direct")
    torch.cuda.synchronize()
    T, U = oracle.gemm(A, oracle.dequant_q4(q, N, K), "f16", trans_b=True, epi="bias_gelu",
                       bias=bias)
    assert_close(C, T, U)


def test_fused_k_zero_full_tiles_is_the_bias():
    # K = 0 with M and N multiples of every tile: no weights, C = bias (beta
    # is 0 here); nothing may load a first K stage
    M, N = 512, 512
    r = np.random.Generator(np.random.PCG64(5500))
    bias_bits = inputs.to_bits(r.uniform(-1, 1, N), "f16")
    A = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    q = torch.empty(0, dtype=torch.uint8, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dge.gemm_q4_f16(A, q, N, 0, C, epi="bias", bias=to_dev(bias_bits, "f16"))
    torch.cuda.synchronize()
    want = np.broadcast_to(oracle.decode(bias_bits, "f16").astype(np.float32), (M, N))
    assert np.array_equal(C.cpu().numpy(), want)


def test_fused_ragged_shape_falls_back_through_the_workspace():
    # M, N not multiples of any tile: the weights are expanded into the workspace
    M, N, K = 33, 70, 256
    q = _unit_scale_q4(N, K, 5400)
    r = np.random.Generator(np.random.PCG64(5401))
    A = inputs.to_bits(r.integers(-4, 5, (M, K)).astype(float), "f16")
    T, _, _ = oracle.prefill(A, q, N, K, want_U=False)
    with pytest.raises(dge.GemmError) as e:
        dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, out_dtype=torch.float32)
    assert e.value.status == 3  # GEMM_ERR_WORKSPACE
    with pytest.raises(dge.GemmError) as e:
        dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, out_dtype=torch.float32,
                        algo="mfma_direct")
    assert e.value.status == 2  # GEMM_ERR_NOT_SUPPORTED: the fused kernel was required
    ws = torch.empty(N * K // 2, dtype=torch.float32, device="cuda")
    C = dge.gemm_q4_f16(to_dev(A, "f16"), _q(q), N, K, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert_bits(C, T)
    assert np.array_equal(bits_of(ws.view(torch.float16)[: N * K].view(N, K)),
                          oracle.dequant_q4(q, N, K))
