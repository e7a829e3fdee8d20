"""Pins for the oracle's block-scaled GEMM against results fixed independently
of it: hand-worked closed forms, exact rational brute force, integer-valued
inputs against int64 arithmetic, a numpy fp64 BLAS product of the dequantised
operands, an identity weight that exposes every code, and the invariants the
definition implies (sign, linearity, row / column-block locality, group
additivity).

Definition pinned (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul
for Hopper", sections "Description" and "Numerical safety"):
    C[m,n] = sum_g a_s[m,g] * b_s[n//128,g] * sum_{k in g} A[m,k] * B[n,k]
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests._cases import exact_int_reference, golden_cases, torch_decode

NON_NAN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_handworked_cases(case):
    C = oracle.block_gemm(case["A"], case["a_s"], case["B"], case["b_s"])
    assert np.array_equal(C, case["C"])
    if case["C_bits"]:
        for dt, hexbits in case["C_bits"].items():
            assert int(oracle.round_bits(C, dt)[0, 0]) == int(hexbits, 16), dt


def _exact(A, a_s, B, b_s):
    """Exact rational C by brute force (torch decode -> Fraction)."""
    dA, dB = torch_decode(A), torch_decode(B)
    M, K = A.shape
    N = B.shape[0]
    G = (K + 127) // 128
    out = [[Fraction(0)] * N for _ in range(M)]
    terms = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(G):
                ks = range(128 * g, min(128 * g + 128, K))
                p = sum((Fraction(float(dA[m, k])) * Fraction(float(dB[n, k])) for k in ks), Fraction(0))
                s = Fraction(float(a_s[m, g])) * Fraction(float(b_s[n // 128, g]))
                acc += p * s
                terms[m, n] += float(sum(abs(dA[m, k] * dB[n, k]) for k in ks)) * abs(float(s))
            out[m][n] = acc
    return out, terms


@pytest.mark.parametrize("seed,M,N,K", [(1, 3, 4, 128), (2, 4, 3, 256), (3, 2, 2, 200), (4, 1, 130, 128)])
def test_brute_force_exact_rational(seed, M, N, K):
    rng = np.random.default_rng(seed)
    A = rng.choice(NON_NAN, size=(M, K)).astype(np.uint8)
    B = rng.choice(NON_NAN, size=(N, K)).astype(np.uint8)
    G, NB = (K + 127) // 128, (N + 127) // 128
    a_s = (rng.standard_normal((M, G)) * np.exp2(rng.integers(-12, 4, (M, G)))).astype(np.float32)
    b_s = (rng.standard_normal((NB, G)) * np.exp2(rng.integers(-12, 4, (NB, G)))).astype(np.float32)
    C = oracle.block_gemm(A, a_s, B, b_s)
    exact, terms = _exact(A, a_s, B, b_s)
    bound = (2 * G + 2) * 2.0 ** -53 * terms
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(C[m, n])) - exact[m][n]) <= Fraction(float(bound[m, n])), (m, n)


def test_integer_mode_is_exact():
    for seed, (M, N, K) in enumerate([(5, 7, 128), (33, 130, 512), (17, 256, 1024)]):
        d = workloads.make_exact_inputs(M, N, K, seed)
        C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        ref16 = exact_int_reference(d, K)
        assert np.array_equal(C * 16, ref16.astype(np.float64)), (M, N, K)
        assert np.abs(ref16).max() < 2 ** 53


def test_integer_mode_with_outlier_rows_is_exact():
    M, N, K = 40, 256, 4096
    d = workloads.make_exact_inputs(M, N, K, 9, u_range=(-2, 0), v_range=(-2, 0),
                                    outlier_rows=[3, 17], outlier_u=3)
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    assert np.array_equal(C * 16, exact_int_reference(d, K).astype(np.float64))


def _dequant_blas(A, a_s, B, b_s):
    K = A.shape[1]
    N = B.shape[0]
    As = torch_decode(A) * np.repeat(a_s.astype(np.float64), 128, axis=1)[:, :K]
    bs_full = np.repeat(np.repeat(b_s.astype(np.float64), 128, axis=0)[:N], 128, axis=1)[:, :K]
    Bs = torch_decode(B) * bs_full
    C = As @ Bs.T
    terms = np.abs(As) @ np.abs(Bs).T
    return C, terms


@pytest.mark.parametrize("M,N,K", [(37, 300, 512), (64, 512, 1024), (3, 1000, 256)])
def test_matches_numpy_blas_of_dequantised_operands(M, N, K):
    d = workloads.make_inputs(M, N, K, seed=M + N)
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    ref, terms = _dequant_blas(d["A"], d["a_s"], d["B"], d["b_s"])
    assert np.all(np.abs(C - ref) <= 4 * K * 2.0 ** -53 * terms + 1e-300)
    # a transposed or swapped operand would be far off, not within rounding
    assert not np.allclose(C[:, :-1], ref[:, 1:])


def test_unit_scales_one_group_equal_plain_fp8_matmul():
    rng = np.random.default_rng(21)
    A = rng.choice(NON_NAN, size=(20, 128)).astype(np.uint8)
    B = rng.choice(NON_NAN, size=(150, 128)).astype(np.uint8)
    C = oracle.block_gemm(A, np.ones((20, 1), np.float32), B, np.ones((2, 1), np.float32))
    assert np.array_equal(C, torch_decode(A) @ torch_decode(B).T)   # both exact


def test_identity_weight_exposes_every_code():
    K = N = 256
    codes = np.concatenate([NON_NAN, np.zeros(2, np.uint8)])          # 254 codes + 2 zeros
    rng = np.random.default_rng(5)
    A = np.stack([codes, rng.permutation(codes)]).astype(np.uint8)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), np.arange(K)] = 0x38                               # 1.0 on the diagonal
    a_s = np.array([[0.5, 3.0], [1.25, 2.0 ** -7]], np.float32)
    C = oracle.block_gemm(A, a_s, B, np.ones((2, 2), np.float32))
    expect = torch_decode(A) * np.repeat(a_s.astype(np.float64), 128, axis=1)
    assert np.array_equal(C, expect)


def test_zero_scale_or_zero_weight_gives_positive_zero():
    d = workloads.make_inputs(8, 256, 256, seed=3)
    C = oracle.block_gemm(d["A"], np.zeros_like(d["a_s"]), d["B"], d["b_s"])
    assert np.all(C == 0) and not np.signbit(C).any()
    C = oracle.block_gemm(d["A"], d["a_s"], np.zeros_like(d["B"]), d["b_s"])
    assert np.all(C == 0) and not np.signbit(C).any()


def test_sign_flip_negates_exactly():
    d = workloads.make_inputs(16, 384, 512, seed=4)
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    Cn = oracle.block_gemm(d["A"] ^ 0x80, d["a_s"], d["B"], d["b_s"])
    assert np.array_equal(Cn, -C)


def test_power_of_two_scale_linearity():
    d = workloads.make_inputs(16, 256, 512, seed=6)
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    for p in (-3, 5):
        Cp = oracle.block_gemm(d["A"], d["a_s"] * np.float32(2.0 ** p), d["B"], d["b_s"])
        assert np.array_equal(Cp, C * 2.0 ** p)
        Cq = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"] * np.float32(2.0 ** p))
        assert np.array_equal(Cq, C * 2.0 ** p)


def test_row_and_column_block_locality():
    M, N, K = 12, 384, 512
    d = workloads.make_inputs(M, N, K, seed=7)
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    a2 = d["a_s"].copy()
    a2[5, 2] *= 3
    C2 = oracle.block_gemm(d["A"], a2, d["B"], d["b_s"])
    changed_rows = np.nonzero(np.any(C2 != C, axis=1))[0]
    assert list(changed_rows) == [5]
    b2 = d["b_s"].copy()
    b2[1, 3] *= 3
    C3 = oracle.block_gemm(d["A"], d["a_s"], d["B"], b2)
    changed_cols = np.nonzero(np.any(C3 != C, axis=0))[0]
    assert changed_cols.size and changed_cols.min() == 128 and changed_cols.max() == 255


def test_group_additivity():
    M, N, K = 10, 200, 512
    d = workloads.make_inputs(M, N, K, seed=8)
    G = K // 128
    C = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    parts = []
    for g in range(G):
        a = np.zeros_like(d["a_s"])
        a[:, g] = d["a_s"][:, g]
        parts.append(oracle.block_gemm(d["A"], a, d["B"], d["b_s"]))
    total = sum(parts)
    _, terms = _dequant_blas(d["A"], d["a_s"], d["B"], d["b_s"])
    assert np.all(np.abs(total - C) <= 4 * G * 2.0 ** -53 * terms)


def test_tolerance_formula_landmarks():
    C_ref = np.array([[1.0, -3.0], [0.0, 1000.0]])
    rms = np.sqrt(np.mean(C_ref ** 2))
    tol = oracle.tolerance(C_ref, "bf16")
    assert np.allclose(tol, 2 * np.array([[2 ** -7, 2 ** -6], [2.0 ** -133, 4.0]]) + 1e-3 * rms)
