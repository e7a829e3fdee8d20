"""The automatic dispatch on random shapes: 48 seeded (M, N, K) draws across
every variant's region (small and large M, K = 256 and longer, ragged M and
N), each through fp8_block_gemm with the dispatcher's own choice, compared
with the oracle -- within tolerance on the standard recipe, bit for bit on
integer-valued inputs with power-of-two scales (every FP32 partial exact).
(FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for Hopper",
section "Description": every shape routed by (M, N, K) to one of the paths.)
"""
import numpy as np
import pytest

import block_scaled_fp8_gemm_amd as fbg
import oracle
import workloads
from tests._gpu import assert_bitwise, assert_within_tolerance, run, to_dev

pytestmark = pytest.mark.gpu


def shapes():
    rng = np.random.default_rng(2024)
    out = []
    while len(out) < 48:
        M = int(rng.choice([rng.integers(1, 33), rng.integers(33, 300), rng.integers(300, 1100)]))
        N = int(rng.choice([rng.integers(1, 200), rng.integers(200, 1200), rng.integers(1200, 2600)]))
        K = int(128 * rng.choice([1, 2, 2, 3, 8, 16, 24, 96]))
        if M * N * K <= 3e8:
            out.append((M, N, K))
    return out


SHAPES = shapes()


def test_the_draws_reach_every_variant():
    names = {fbg.plan(M, N, K)["variant_name"] for M, N, K in SHAPES}
    assert names == {"generic", "short_k256", "swap_ab", "swap_ab_splitk"}, names


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_auto_dispatch_random_shape(gpu, i):
    M, N, K = SHAPES[i]
    p = fbg.plan(M, N, K)
    what = f"{M}x{N}x{K} -> {p['variant_name']} cfg {p['config']} S={p['split_k']}"
    if i % 2 == 0:
        d = workloads.make_inputs(M, N, K, seed=500 + i)
        ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        assert_within_tolerance(run(fbg, to_dev(d)), ref, "bf16", what)
    else:
        d = workloads.make_exact_inputs(M, N, K, seed=500 + i)
        ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        assert_bitwise(run(fbg, to_dev(d), "fp32"), ref, "fp32", what)
