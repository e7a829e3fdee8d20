"""fp8_block_gemm_noalloc (the entry point for callers that cannot allocate:
split-K partials and counters in the library's static per-GPU scratch)
against fp8_block_gemm_ex with a caller-owned workspace: the same plan and
kernels, so the outputs must be equal bit for bit; checked on two calls in a
row, the second with a smaller input, and against the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_within_tolerance, to_dev

pytestmark = pytest.mark.gpu


def _ex(gpu, dd, M, N, K, out_dtype, variant="auto", split_k=0):
    ws = torch.zeros(max(gpu.workspace_size(M, N, K, variant, split_k), 16), dtype=torch.uint8, device="cuda:0")
    return gpu.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out_dtype=out_dtype, workspace=ws, variant=variant,
                    split_k=split_k)


def test_noalloc_matches_the_workspace_entry_point(gpu):
    # a decode shape the dispatcher splits in four, then a smaller one that
    # also splits, then a forced split of a ragged shape: each call's output
    # equals fp8_block_gemm_ex's with a caller workspace, bit for bit
    cases = [((32, 512, 16384), "auto", 0, torch.bfloat16),
             ((16, 512, 16384), "auto", 0, torch.bfloat16),
             ((50, 300, 2048), "swap_ab_splitk", 3, torch.float32)]
    for (M, N, K), variant, split_k, od in cases:
        p = gpu.plan(M, N, K, od, torch.cuda.get_device_properties(0).multi_processor_count, variant, split_k)
        assert p["split_k"] > 1, (M, N, K)
        d = workloads.make_inputs(M, N, K, seed=M + N)
        dd = to_dev(d)
        C = torch.full((M, N), float("nan"), dtype=od, device="cuda:0")
        gpu.gemm_noalloc(dd["A"], dd["a_s"], dd["B"], dd["b_s"], C, variant=variant, split_k=split_k)
        want = _ex(gpu, dd, M, N, K, od, variant, split_k)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.uint8), want.view(torch.uint8)), (M, N, K)
        out = {torch.bfloat16: "bf16", torch.float32: "fp32"}[od]
        assert_within_tolerance(C, oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"]), out, f"{M},{N},{K}")


def test_noalloc_repeated_calls_on_a_stream(gpu):
    # calls ordered on one stream reuse the scratch: each leaves the counters
    # zero for the next (a wrong count would make a tile skip its reduction)
    M, N, K = 32, 512, 16384
    d = workloads.make_inputs(M, N, K, seed=5)
    dd = to_dev(d)
    want = _ex(gpu, dd, M, N, K, torch.bfloat16)
    s = torch.cuda.Stream()
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0") for _ in range(6)]
    with torch.cuda.stream(s):
        for o in outs:
            gpu.gemm_noalloc(dd["A"], dd["a_s"], dd["B"], dd["b_s"], o, stream=s)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.uint8), want.view(torch.uint8))


def test_noalloc_rejects_a_split_beyond_its_scratch(gpu):
    # 4096 x 4096 in 32 x 16 tiles split 4 ways: 128 x 256 tiles, 32 MiB of partials
    M, N, K = 4096, 4096, 1024
    dd = {"A": torch.zeros((M, K), dtype=torch.float8_e4m3fn, device="cuda:0"),
          "a_s": torch.ones((M, K // 128), device="cuda:0"),
          "B": torch.zeros((N, K), dtype=torch.float8_e4m3fn, device="cuda:0"),
          "b_s": torch.ones((N // 128, K // 128), device="cuda:0")}
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(gpu.FP8BGError) as e:
        gpu.gemm_noalloc(dd["A"], dd["a_s"], dd["B"], dd["b_s"], C, variant="swap_ab_splitk", split_k=4)
    assert e.value.status == gpu.SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())          # nothing launched
    # the plain entry points still work after the rejected call
    e2 = workloads.make_inputs(16, 256, 512, seed=3)
    de = to_dev(e2)
    C2 = torch.empty((16, 256), dtype=torch.float32, device="cuda:0")
    gpu.gemm_noalloc(de["A"], de["a_s"], de["B"], de["b_s"], C2)
    torch.cuda.synchronize()
    assert_within_tolerance(C2, oracle.block_gemm(e2["A"], e2["a_s"], e2["B"], e2["b_s"]), "fp32", "small")
