"""The largest K the boundary accepts (2^24 - 128: a 256-row tile's bytes must
end below 2^32, the reach of the kernels' 32-bit buffer offsets), with 256 real
rows in a tile, so the generic 256 x 256 tiles address bytes up to 128 x 256
bytes short of 4 GiB from the tile's first row.  (At K = 2^24 the last dword
of such a tile read as zero; the boundary now refuses that K.)
Integer-valued codes in the first, a middle and the last group of every row
(zeros elsewhere) and power-of-two scales make every partial exact, so the
sampled outputs must equal the oracle bit for bit.  (FlagGems-vllm PR #693,
"feat: optimize w8a8 block fp8 matmul for Hopper", section "Numerical
safety": the guard admits any K that is a multiple of 128.)  Also an output
of more than 2^31 elements.
"""
import numpy as np
import pytest

import block_scaled_fp8_gemm_amd as fbg
import oracle
import workloads
from tests._gpu import bits, run, to_dev

pytestmark = pytest.mark.gpu

K = (1 << 24) - 128
G = K // 128
EDGE = [0, 1, 127, 128, 254, 255]


def operands(M, N, seed):
    rng = np.random.default_rng(seed)

    def codes(rows):
        X = np.zeros((rows, K), np.uint8)
        for g in (0, G // 2, G - 1):
            X[:, 128 * g:128 * (g + 1)] = workloads.e4m3_code_of_int(rng.integers(-4, 5, size=(rows, 128)))
        return X

    A, B = codes(M), codes(N)
    a_s = np.ldexp(np.float32(1.0), rng.integers(-2, 2, size=(M, G))).astype(np.float32)
    b_s = np.ldexp(np.float32(1.0), rng.integers(-2, 2, size=((N + 127) // 128, G))).astype(np.float32)
    return {"A": A, "a_s": a_s, "B": B, "b_s": b_s}


@pytest.mark.parametrize("M,N", [(256, 16), (16, 256)])
@pytest.mark.parametrize("variant,cfg", [("generic", 8), ("generic", 3), ("auto", None)])
def test_largest_k_bitwise_on_edge_rows(gpu, M, N, variant, cfg):
    assert gpu.plan(M, N, K)["variant"] >= 0  # the boundary admits this K
    d = operands(M, N, seed=M + 7 * N)
    C = run(fbg, to_dev(d), "fp32", variant=variant, cfg=cfg)
    got = bits(C, "fp32")
    rows = [r for r in EDGE if r < M]
    cols = [c for c in EDGE if c < N]
    for c in cols:
        ref = oracle.block_gemm(d["A"][rows], d["a_s"][rows], d["B"][c:c + 1], d["b_s"][c // 128:c // 128 + 1])
        want = oracle.round_bits(ref, "fp32")[:, 0]
        assert np.array_equal(got[rows, c], want), (variant, cfg, M, N, c, got[rows, c], want)


def test_output_past_2_to_31_elements(gpu):
    """C of 2^32 elements (M = 2^17, N = 2^15): every store index past 2^31
    must be formed in 64 bits.  Sampled rows, bit for bit in exact mode."""
    M, N, K2 = 1 << 17, 1 << 15, 128
    d = workloads.make_exact_inputs(M, N, K2, seed=5)
    C = run(fbg, to_dev(d), "bf16")
    rows = [0, 1, 65535, 65536, M - 2, M - 1]
    got = bits(C[rows], "bf16")
    del C
    ref = oracle.block_gemm(d["A"][rows], d["a_s"][rows], d["B"], d["b_s"])
    assert np.array_equal(got, oracle.round_bits(ref, "bf16"))
