"""Pins for the oracle GEMM, independent of the oracle itself.

* brute force in exact rational arithmetic on tiny shapes (where binary64
  accumulation is provably exact for fp16 inputs, and within K*2^-53*U for
  fp32 and bf16 inputs);
* small-integer inputs against an int64 triple product at any K;
* identity and permutation matrices (exact column/row movement);
* closed forms (ones * ones = K, A=1 and B_kj = k gives K(K-1)/2);
* the trans_b = 0 / trans_b = 1 invariant and thread-count invariance;
* exact linearity in alpha and beta with integer data.
Shapes are non-square with M, N, K all distinct, so a transposed operand or a
swapped index fails.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_engineering_amd import inputs


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _frac_gemm(Ad, Bd):
    M, K = Ad.shape
    N = Bd.shape[1]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(Ad[i, k]) * Fraction(Bd[k, j])
            out[i][j] = s
    return out


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (5, 2, 32), (1, 1, 1), (4, 6, 17)])
@pytest.mark.parametrize("trans_b", [False, True])
def test_fp16_exact_against_fractions(M, N, K, trans_b):
    r = _rng(100 + M * 31 + N * 7 + K)
    A = inputs.to_bits(r.uniform(-1, 1, (M, K)), "f16")
    Bkn = inputs.to_bits(r.uniform(-1, 1, (K, N)), "f16")
    B = np.ascontiguousarray(Bkn.T) if trans_b else Bkn
    T, U = oracle.gemm(A, B, "f16", trans_b=trans_b)
    Ad = A.view(np.float16).astype(np.float64)
    Bd = Bkn.view(np.float16).astype(np.float64)
    exact = _frac_gemm(Ad, Bd)
    for i in range(M):
        for j in range(N):
            assert Fraction(T[i, j]) == exact[i][j]
            ua = sum(abs(Fraction(Ad[i, k]) * Fraction(Bd[k, j])) for k in range(K))
            assert Fraction(U[i, j]) == ua


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp32_bf16_against_fractions_within_bound(dtype):
    M, N, K = 4, 3, 40
    r = _rng(200)
    A = inputs.to_bits(r.uniform(-1, 1, (M, K)), dtype)
    B = inputs.to_bits(r.uniform(-1, 1, (K, N)), dtype)
    T, U = oracle.gemm(A, B, dtype)
    Ad = oracle.decode(A, dtype)
    Bd = oracle.decode(B, dtype)
    if dtype == "f32":
        assert np.array_equal(Ad, A.view(np.float32).astype(np.float64))
    exact = _frac_gemm(Ad, Bd)
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(T[i, j]) - exact[i][j])
            assert err <= Fraction(K) * Fraction(2) ** -53 * Fraction(U[i, j])


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("trans_b", [False, True])
def test_small_integers_against_int64(dtype, trans_b):
    M, N, K = 37, 29, 1000
    r = _rng(300)
    Ai = r.integers(-4, 5, (M, K))
    Bi = r.integers(-4, 5, (K, N))
    A = inputs.to_bits(Ai.astype(np.float64), dtype)
    Bkn = inputs.to_bits(Bi.astype(np.float64), dtype)
    B = np.ascontiguousarray(Bkn.T) if trans_b else Bkn
    T, U = oracle.gemm(A, B, dtype, trans_b=trans_b)
    want = Ai.astype(np.int64) @ Bi.astype(np.int64)
    assert np.array_equal(T, want.astype(np.float64))
    assert np.array_equal(U, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


@pytest.mark.parametrize("trans_b", [False, True])
def test_identity_and_permutation(trans_b):
    M, K = 19, 24
    r = _rng(400)
    A = inputs.to_bits(r.uniform(-1, 1, (M, K)), "f16")
    I = inputs.to_bits(np.eye(K), "f16")
    T, _ = oracle.gemm(A, I, "f16", trans_b=trans_b)
    assert np.array_equal(T, A.view(np.float16).astype(np.float64))
    perm = r.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0  # (A P)[:, j] = A[:, perm[j]]
    Pb = inputs.to_bits(P, "f16")
    B = np.ascontiguousarray(Pb.T) if trans_b else Pb
    T, _ = oracle.gemm(A, B, "f16", trans_b=trans_b)
    assert np.array_equal(T, A.view(np.float16).astype(np.float64)[:, perm])
    # permutation on the left moves rows of B
    N = 13
    Bm = inputs.to_bits(r.uniform(-1, 1, (K, N)), "f16")
    Pl = np.zeros((K, K))
    Pl[np.arange(K), perm] = 1.0  # (P B)[i, :] = B[perm[i], :]
    T, _ = oracle.gemm(inputs.to_bits(Pl, "f16"), Bm, "f16")
    assert np.array_equal(T, Bm.view(np.float16).astype(np.float64)[perm, :])


def test_closed_forms():
    for K in (1, 7, 256, 2048):
        A = inputs.to_bits(np.ones((3, K)), "f16")
        B = inputs.to_bits(np.ones((K, 5)), "f16")
        T, _ = oracle.gemm(A, B, "f16")
        assert np.all(T == K)
    K = 4096
    A = inputs.to_bits(np.ones((2, K)), "f32")
    B = inputs.to_bits(np.repeat(np.arange(K, dtype=np.float64)[:, None], 3, axis=1), "f32")
    T, _ = oracle.gemm(A, B, "f32")
    assert np.all(T == K * (K - 1) / 2)


def test_trans_b_invariant_and_threads_bitwise():
    M, N, K = 41, 23, 300
    A, B = (inputs.normal((M, K), "f16", 9, 1), inputs.normal((K, N), "f16", 9, 2))
    T0, U0 = oracle.gemm(A, B, "f16", threads=1)
    T1, U1 = oracle.gemm(A, np.ascontiguousarray(B.T), "f16", trans_b=True, threads=5)
    assert np.array_equal(T0, T1) and np.array_equal(U0, U1)


def test_alpha_beta_linearity_exact():
    M, N, K = 11, 17, 64
    r = _rng(500)
    Ai, Bi, Ci = r.integers(-4, 5, (M, K)), r.integers(-4, 5, (K, N)), r.integers(-50, 51, (M, N))
    A = inputs.to_bits(Ai.astype(float), "f16")
    B = inputs.to_bits(Bi.astype(float), "f16")
    S = (Ai @ Bi).astype(np.float64)
    for alpha in (1.0, -1.0, 2.0, 0.5, 0.0):
        for beta in (0.0, 1.0, -2.0, 0.5):
            T, _ = oracle.gemm(A, B, "f16", alpha=alpha, beta=beta, C_old=Ci.astype(float))
            assert np.array_equal(T, alpha * S + beta * Ci)


def test_beta_zero_never_reads_c():
    A, B = inputs.square256()
    C_old = np.full((256, 256), np.nan)
    T, _ = oracle.gemm(A[:8], B, "f16", beta=0.0, C_old=C_old[:8])
    assert np.all(np.isfinite(T))


def test_k_zero_gives_beta_c():
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((0, 4), dtype=np.uint16)
    C = np.arange(12, dtype=np.float64).reshape(3, 4)
    T, U = oracle.gemm(A, B, "f16", beta=2.0, C_old=C)
    assert np.array_equal(T, 2 * C) and np.all(U == 0)


def test_bf16_output_rounding_exceeds_1e3_by_construction():
    # Why bf16 outputs get the widened normwise bound: rounding an exact
    # result to bf16 alone already gives ~1.1e-3 normwise relative error.
    from oracle import compare
    A, B = inputs.square256()
    T, _ = oracle.gemm(A[:64], B, "f16")
    Cb = oracle.decode(oracle.encode(T, "bf16"), "bf16")
    e = compare.normwise_rel_err(Cb, T)
    assert 1e-3 < e < compare.normwise_tol("bf16")
    Ch = oracle.decode(oracle.encode(T, "f16"), "f16")
    assert compare.normwise_rel_err(Ch, T) < 1e-3 / 2
