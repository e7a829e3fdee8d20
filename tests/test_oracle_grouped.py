"""Pins for the oracle's grouped (mixture-of-experts) block-scaled GEMM: each
token row is multiplied by the weight of the expert whose row range holds
it, with that expert's block scales.  Checked against results fixed
independently of the oracle: exact rational brute force with an explicit
row -> expert lookup, integer-valued inputs against int64 arithmetic, the
relabelling of experts, and the empty-expert and single-expert special
cases.  (MoE-style traffic: FlagGems-vllm PR #693, "feat: optimize w8a8 block
fp8 matmul for Hopper", section "Description"; per-expert weights and token
groups: the MoE kernel page, section "Summary".)
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._cases import torch_decode

NON_NAN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def random_grouped(rng, counts, N, K, scale_exp=(-8, 3)):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    G, NB = (K + 127) // 128, (N + 127) // 128
    A = rng.choice(NON_NAN, size=(M, K)).astype(np.uint8)
    B = rng.choice(NON_NAN, size=(E, N, K)).astype(np.uint8)
    a_s = (rng.random((M, G)) * np.exp2(rng.integers(*scale_exp, (M, G)))).astype(np.float32)
    b_s = (rng.random((E, NB, G)) * np.exp2(rng.integers(*scale_exp, (E, NB, G)))).astype(np.float32)
    return A, a_s, B, b_s, offsets


def test_brute_force_with_explicit_expert_lookup():
    rng = np.random.default_rng(1)
    A, a_s, B, b_s, off = random_grouped(rng, [2, 0, 1, 3], 3, 256)
    C = oracle.grouped_gemm(A, a_s, B, b_s, off)
    dA = torch_decode(A)
    for m in range(A.shape[0]):
        e = int(np.searchsorted(off, m, side="right") - 1)      # the expert whose rows hold m
        dB = torch_decode(B[e])
        for n in range(B.shape[1]):
            exact = Fraction(0)
            for g in range(2):
                p = sum((Fraction(float(dA[m, k])) * Fraction(float(dB[n, k])) for k in range(128 * g, 128 * g + 128)),
                        Fraction(0))
                exact += p * Fraction(float(a_s[m, g])) * Fraction(float(b_s[e, n // 128, g]))
            assert abs(C[m, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact))), (m, n)


def test_integer_mode_against_int64():
    rng = np.random.default_rng(2)
    counts = [5, 0, 17, 1, 9]
    E, N, K = len(counts), 140, 384
    off = np.concatenate([[0], np.cumsum(counts)])
    M, G = int(off[-1]), K // 128
    Ai = rng.integers(-4, 5, (M, K))
    Bi = rng.integers(-4, 5, (E, N, K))
    enc = np.vectorize(oracle.e4m3_encode)
    A = enc(Ai.astype(np.float64)).astype(np.uint8)
    B = enc(Bi.astype(np.float64)).astype(np.uint8)
    ua = rng.integers(-2, 2, (M, G))
    ub = rng.integers(-2, 2, (E, (N + 127) // 128, G))
    a_s, b_s = np.exp2(ua).astype(np.float32), np.exp2(ub).astype(np.float32)
    C = oracle.grouped_gemm(A, a_s, B, b_s, off)
    # int64 reference in units of 2^-4 (the smallest scale product)
    want = np.zeros((M, N), dtype=np.int64)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        for g in range(G):
            p = Ai[r0:r1, 128 * g:128 * g + 128] @ Bi[e, :, 128 * g:128 * g + 128].T
            sh = ua[r0:r1, g][:, None] + ub[e, np.arange(N) // 128, g][None, :] + 4
            want[r0:r1] += p * (1 << sh)
    assert np.array_equal(C, want.astype(np.float64) / 16.0)


def test_relabelling_experts_permutes_rows():
    rng = np.random.default_rng(3)
    counts = [3, 4, 0, 2]
    A, a_s, B, b_s, off = random_grouped(rng, counts, 130, 256)
    C = oracle.grouped_gemm(A, a_s, B, b_s, off)
    perm = [2, 0, 3, 1]                       # new expert i is old expert perm[i]
    segs = [np.arange(off[e], off[e + 1]) for e in range(len(counts))]
    rows = np.concatenate([segs[p] for p in perm])
    off2 = np.concatenate([[0], np.cumsum([counts[p] for p in perm])])
    C2 = oracle.grouped_gemm(A[rows], a_s[rows], B[perm], b_s[perm], off2)
    assert np.array_equal(C2, C[rows])


def test_single_expert_is_the_plain_gemm_and_empty_experts_are_ignored():
    rng = np.random.default_rng(4)
    A, a_s, B, b_s, off = random_grouped(rng, [7], 200, 384)
    assert np.array_equal(oracle.grouped_gemm(A, a_s, B, b_s, off), oracle.block_gemm(A, a_s, B[0], b_s[0]))
    # the same tokens with empty experts around them
    Bx = np.stack([rng.choice(NON_NAN, size=B.shape[1:]).astype(np.uint8), B[0],
                   rng.choice(NON_NAN, size=B.shape[1:]).astype(np.uint8)])
    bx = np.stack([b_s[0] * 3, b_s[0], b_s[0] * 5])
    C = oracle.grouped_gemm(A, a_s, Bx, bx, [0, 0, 7, 7])
    assert np.array_equal(C, oracle.block_gemm(A, a_s, B[0], b_s[0]))


def test_rejects_bad_offsets():
    rng = np.random.default_rng(5)
    A, a_s, B, b_s, off = random_grouped(rng, [2, 3], 16, 128)
    for bad in ([0, 3, 2], [1, 2, 5], [0, 2, 6], [0, 5]):
        with pytest.raises(ValueError):
            oracle.grouped_gemm(A, a_s, B, b_s, bad)
