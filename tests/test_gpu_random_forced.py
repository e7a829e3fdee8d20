"""Seeded random draws of (shape, variant, tile configuration, split, output
dtype), dense and grouped, on integer-valued inputs with power-of-two scales
(every FP32 partial exact, so every summation order gives one result): each
launch must equal the oracle bit for bit.  Forced configurations that a
shape's guard refuses return UNSUPPORTED and are skipped; the draws are
fixed, so the same cases run every time.  (FlagGems-vllm PR #693, "feat:
optimize w8a8 block fp8 matmul for Hopper", sections "Description" and
"Numerical safety": every path computes the same block-scaled product.)
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_gemm_amd as fbg
import oracle
import workloads
from tests._gpu import TORCH_OUT, assert_bitwise, forced_config, run, to_dev

pytestmark = pytest.mark.gpu

CHUNK = 10


def dense_cases(n=400, seed=97):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300), rng.integers(300, 700)]))
        N = int(rng.choice([rng.integers(1, 300), rng.integers(300, 1700)]))
        K = int(128 * rng.choice([1, 2, 2, 3, 5, 8, 16, 24, 40]))
        if M * N * K > 2e8:
            continue
        kind = int(rng.integers(0, 5))
        if kind == 0:
            v = ("auto", None, 0)
        elif kind == 1:
            v = ("generic", int(rng.integers(0, 12)), 0)
        elif kind == 2:
            v = ("swap_ab", int(rng.integers(0, 24)), 0)
        elif kind == 3:
            v = ("swap_ab_splitk", int(rng.integers(0, 23)), int(rng.integers(2, 9)))
        elif K == 256:
            v = ("short_k256", int(rng.integers(0, 16)), 0)
        else:
            continue
        out.append((M, N, K) + v + (str(rng.choice(["bf16", "fp16", "fp32"])), int(rng.integers(1 << 30))))
    return out


def grouped_cases(n=200, seed=98):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 2, 5, 17, 70]))
        counts = [int(rng.choice([0, rng.integers(1, 20), rng.integers(20, 140), rng.integers(140, 400)]))
                  for _ in range(E)]
        N = int(rng.choice([rng.integers(1, 300), rng.integers(300, 700)]))
        K = int(128 * rng.choice([1, 2, 3, 8, 9]))
        if sum(counts) * N * K > 2e8 or E * N * K > 1e8:
            continue
        cfg = None if rng.integers(0, 4) == 0 else int(rng.integers(0, 19))
        out.append((counts, N, K, cfg, str(rng.choice(["bf16", "fp16", "fp32"])), int(rng.integers(1 << 30))))
    return out


def single_stage_cases(n=300, seed=99):
    """The single-stage swap-AB tiles (configurations 22 and 23: every load of
    a workgroup in flight at once, weight rows issued before activation rows),
    on ragged M and N and on group counts that leave partial chunks."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(1, 20), rng.integers(20, 130), rng.integers(130, 400)]))
        N = int(rng.choice([rng.integers(1, 200), rng.integers(200, 1100)]))
        K = int(128 * rng.integers(1, 41))
        if M * N * K > 2e8:
            continue
        out.append((M, N, K, "swap_ab", int(rng.choice([22, 23])), 0,
                    str(rng.choice(["bf16", "fp16", "fp32"])), int(rng.integers(1 << 30))))
    return out


DENSE = dense_cases()
SINGLE = single_stage_cases()
GROUPED = grouped_cases()


def test_the_draws_cover_every_variant_and_many_configurations():
    assert {c[3] for c in DENSE} == {"auto", "generic", "swap_ab", "swap_ab_splitk", "short_k256"}
    assert len({(c[3], c[4]) for c in DENSE}) >= 60
    assert len({c[3] for c in GROUPED}) >= 15


def run_dense_chunk(cases):
    ran = 0
    for M, N, K, variant, cfg, S, out, seed in cases:
        what = f"{M}x{N}x{K} {variant} cfg={cfg} S={S} {out} seed={seed}"
        d = workloads.make_exact_inputs(M, N, K, seed=seed)
        try:
            C = run(fbg, to_dev(d), out, variant=variant, split_k=S, cfg=cfg)
        except fbg.FP8BGError as e:
            assert e.status == fbg.UNSUPPORTED, what
            continue
        assert_bitwise(C, oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"]), out, what)
        ran += 1
    return ran


@pytest.mark.parametrize("chunk", range(len(DENSE) // CHUNK))
def test_random_forced_dense_bitwise(gpu, chunk):
    assert run_dense_chunk(DENSE[chunk * CHUNK:(chunk + 1) * CHUNK]) > 0


@pytest.mark.parametrize("chunk", range(len(SINGLE) // (3 * CHUNK)))
def test_random_single_stage_bitwise(gpu, chunk):
    assert run_dense_chunk(SINGLE[chunk * 3 * CHUNK:(chunk + 1) * 3 * CHUNK]) == 3 * CHUNK


@pytest.mark.parametrize("chunk", range(len(GROUPED) // CHUNK))
def test_random_forced_grouped_bitwise(gpu, chunk):
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    for counts, N, K, cfg, out, seed in GROUPED[chunk * CHUNK:(chunk + 1) * CHUNK]:
        what = f"E={len(counts)} counts={counts[:8]} N={N} K={K} cfg={cfg} {out} seed={seed}"
        g = workloads.make_exact_grouped_inputs(counts, N, K, seed=seed)
        with forced_config(cfg):
            C = fbg.grouped_gemm(t(g["A"]).view(torch.float8_e4m3fn), t(g["a_s"]), t(g["B"]).view(torch.float8_e4m3fn),
                                 t(g["b_s"]), t(np.asarray(g["offsets"], dtype=np.int32)), out_dtype=TORCH_OUT[out])
        torch.cuda.synchronize()
        assert_bitwise(C, oracle.grouped_gemm(g["A"], g["a_s"], g["B"], g["b_s"], g["offsets"]), out, what)
