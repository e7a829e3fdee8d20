"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every variant and tile configuration is forced on shapes that span several
tiles and end in ragged tails, for each output dtype, and compared element by
element: within |dC| <= 2 ulp(|C_ref|) + 1e-3 rms(C_ref) on the standard
recipe, bit for bit on integer-valued inputs with power-of-two scales (where
every FP32 partial sum is exact, so any order gives the one correctly rounded
result).  Definition: FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8
matmul for Hopper", sections "Description" and "Numerical safety".
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._cases import golden_cases
from tests._gpu import assert_bitwise, assert_within_tolerance, bits, forced_config, run, to_dev

pytestmark = pytest.mark.gpu

OUTS = ["bf16", "fp16", "fp32"]

# (variant, forced config, M, N, K, split_k): every configuration of every
# variant, several tiles, ragged M and N tails.
TOL_CASES = [
    ("generic", 0, 200, 300, 512, 0),
    ("generic", 0, 129, 257, 384, 0),
    ("generic", 1, 300, 260, 256, 0),
    ("generic", 2, 17, 1000, 256, 0),
    ("generic", 2, 1, 130, 128, 0),
    ("generic", 3, 300, 520, 640, 0),
    ("generic", 3, 513, 257, 256, 0),
    # 256x256 tile with row scales in 8-group chunks: several chunks, the
    # three chunk buffers reused, a partial last chunk, ragged rows.
    ("generic", 3, 300, 520, 3200, 0),
    ("generic", 3, 257, 300, 2048, 0),
    ("generic", 4, 200, 300, 1024, 0),
    ("generic", 4, 64, 130, 512, 0),
    ("generic", 4, 1, 100, 256, 0),
    ("generic", 5, 300, 200, 1024, 0),
    ("generic", 5, 65, 515, 384, 0),
    ("generic", 6, 130, 300, 1024, 0),
    ("generic", 6, 64, 33, 256, 0),
    ("generic", 6, 129, 260, 640, 0),
    ("generic", 3, 130, 600, 1152, 0),
    # 256x256 with the mid-group refill: several chunks of row scales, ragged
    # tiles, fewer groups than the ring's prologue, odd group counts
    ("generic", 8, 300, 520, 3200, 0),
    ("generic", 8, 513, 257, 256, 0),
    ("generic", 8, 257, 300, 2048, 0),
    ("generic", 8, 130, 600, 1152, 0),
    ("generic", 8, 300, 520, 640, 0),
    # 2x2 waves of 32x32: two row blocks per wave, ragged tiles, fewer groups
    # than ring slots, more (slots refilled)
    ("generic", 9, 128, 1094, 1024, 0),
    ("generic", 9, 65, 300, 384, 0),
    ("generic", 9, 130, 260, 2560, 0),
    ("generic", 9, 1, 40, 256, 0),
    ("generic", 10, 130, 300, 1024, 0),
    ("generic", 10, 64, 130, 384, 0),
    ("generic", 11, 300, 260, 1024, 0),
    ("generic", 11, 129, 257, 384, 0),
    # 128x256 tile with 8 waves (grouped mid-size experts; forced here dense)
    ("generic", 7, 300, 520, 1024, 0),
    ("generic", 7, 129, 257, 384, 0),
    ("generic", 7, 1, 600, 256, 0),
    ("short_k256", 0, 184, 700, 256, 0),
    ("short_k256", 0, 300, 515, 256, 0),
    ("short_k256", 1, 37, 130, 256, 0),
    ("short_k256", 2, 1, 4096, 256, 0),
    ("short_k256", 3, 30, 333, 256, 0),
    ("short_k256", 4, 16, 600, 256, 0),
    ("short_k256", 5, 64, 515, 256, 0),
    ("short_k256", 6, 20, 260, 256, 0),
    ("short_k256", 7, 128, 300, 256, 0),
    ("short_k256", 7, 184, 130, 256, 0),
    ("swap_ab", 0, 64, 600, 1024, 0),
    ("swap_ab", 1, 100, 333, 512, 0),
    ("swap_ab", 2, 3, 130, 384, 0),
    ("swap_ab", 3, 30, 257, 640, 0),
    ("swap_ab", 4, 40, 260, 640, 0),
    ("swap_ab", 5, 128, 200, 1024, 0),
    ("swap_ab", 5, 200, 130, 512, 0),
    ("swap_ab", 6, 16, 700, 256, 0),
    ("swap_ab", 7, 1, 257, 512, 0),
    ("swap_ab", 8, 64, 200, 1152, 0),
    ("swap_ab", 9, 32, 140, 2048, 0),
    ("swap_ab", 10, 9, 300, 4096, 0),
    ("swap_ab", 11, 16, 130, 2048, 0),
    ("swap_ab", 12, 128, 300, 1024, 0),
    ("swap_ab", 13, 100, 130, 2048, 0),
    ("swap_ab", 14, 64, 260, 1152, 0),
    ("swap_ab", 15, 32, 200, 1024, 0),
    ("swap_ab", 16, 1, 515, 1024, 0),
    ("swap_ab", 17, 7, 600, 640, 0),
    ("swap_ab", 18, 64, 300, 1280, 0),
    ("swap_ab", 19, 50, 130, 1024, 0),
    ("swap_ab", 20, 16, 260, 2048, 0),
    ("swap_ab", 21, 2, 300, 1536, 0),
    ("swap_ab_splitk", 18, 64, 512, 4096, 3),
    ("swap_ab_splitk", 20, 12, 256, 4096, 5),
    ("short_k256", 8, 184, 300, 256, 0),
    ("short_k256", 9, 184, 130, 256, 0),
    ("short_k256", 10, 70, 260, 256, 0),
    ("short_k256", 11, 64, 500, 256, 0),
    ("short_k256", 12, 48, 515, 256, 0),
    ("short_k256", 13, 33, 300, 256, 0),
    ("short_k256", 14, 1, 700, 256, 0),
    ("short_k256", 15, 184, 260, 256, 0),
    ("swap_ab_splitk", 0, 64, 512, 4096, 8),
    ("swap_ab_splitk", 0, 64, 512, 4096, 3),
    ("swap_ab_splitk", 1, 9, 1000, 2048, 16),
    ("swap_ab_splitk", 2, 5, 200, 1024, 2),
    ("swap_ab_splitk", 3, 30, 130, 640, 5),
    ("swap_ab_splitk", 5, 128, 256, 2048, 4),
    ("swap_ab_splitk", 7, 9, 300, 4096, 7),
    ("swap_ab_splitk", 9, 20, 128, 1024, 8),
    ("swap_ab_splitk", 10, 64, 512, 4096, 2),
    ("swap_ab_splitk", 12, 128, 256, 1024, 2),
    ("swap_ab_splitk", 14, 64, 512, 4096, 4),
    # single-stage LDS tile: one chunk covering the range, several chunks (a
    # wave reloading its one area), partial chunks, and splits
    ("swap_ab", 22, 33, 260, 4096, 0),
    ("swap_ab", 22, 64, 300, 4096, 0),
    ("swap_ab", 22, 9, 200, 8192, 0),
    ("swap_ab", 22, 5, 130, 1280, 0),
    ("swap_ab_splitk", 22, 64, 512, 4096, 2),
    ("swap_ab_splitk", 22, 40, 260, 3072, 3),
    # the single-stage tile with 8 activation rows: ragged M (a last tile of
    # 1-7 rows), ragged N, K of fewer groups than the tile's 32, exactly 32,
    # and more (the single area reloaded)
    ("swap_ab", 23, 64, 512, 4096, 0),
    ("swap_ab", 23, 5, 130, 1280, 0),
    ("swap_ab", 23, 70, 300, 2048, 0),
    ("swap_ab", 23, 9, 200, 8192, 0),
    ("swap_ab", 23, 13, 260, 384, 0),
    ("swap_ab", 23, 1, 40, 4096, 0),
]


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("case", TOL_CASES, ids=lambda c: f"{c[0]}-cfg{c[1]}-{c[2]}x{c[3]}x{c[4]}-S{c[5]}")
def test_variant_within_tolerance(gpu, case, out):
    variant, cfg, M, N, K, S = case
    d = workloads.make_inputs(M, N, K, seed=M * 7 + N + K)
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    C = run(gpu, to_dev(d), out, variant, S, cfg)
    assert_within_tolerance(C, ref, out, f"{case} {out}")


EXACT_CASES = [
    ("generic", 0, 150, 300, 1024, 0),
    ("generic", 2, 40, 260, 512, 0),
    ("generic", 3, 260, 300, 768, 0),
    ("generic", 3, 130, 260, 4224, 0),
    ("generic", 8, 260, 300, 768, 0),
    ("generic", 4, 130, 260, 1152, 0),
    ("generic", 9, 130, 260, 1024, 0),
    ("generic", 6, 70, 100, 384, 0),
    ("generic", 8, 130, 260, 4224, 0),
    ("short_k256", 15, 100, 300, 256, 0),
    ("short_k256", 0, 100, 640, 256, 0),
    ("short_k256", 2, 5, 130, 256, 0),
    ("short_k256", 7, 128, 256, 256, 0),
    ("swap_ab", 0, 48, 384, 1024, 0),
    ("swap_ab", 2, 3, 200, 512, 0),
    ("swap_ab", 5, 100, 256, 1024, 0),
    ("swap_ab_splitk", 0, 48, 384, 1024, 2),
    ("swap_ab_splitk", 0, 48, 384, 1024, 8),
    ("swap_ab_splitk", 1, 48, 384, 1024, 3),
    ("swap_ab", 22, 48, 384, 4096, 0),
    ("swap_ab_splitk", 22, 48, 384, 4096, 2),
    ("swap_ab", 23, 48, 384, 4096, 0),
    ("swap_ab", 23, 13, 130, 2560, 0),
]


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("case", EXACT_CASES, ids=lambda c: f"{c[0]}-cfg{c[1]}-{c[2]}x{c[3]}x{c[4]}-S{c[5]}")
def test_exact_mode_bitwise(gpu, case, out):
    variant, cfg, M, N, K, S = case
    d = workloads.make_exact_inputs(M, N, K, seed=M + N)
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    C = run(gpu, to_dev(d), out, variant, S, cfg)
    assert_bitwise(C, ref, out, f"{case} {out}")


def test_exact_mode_outlier_rows_long_k(gpu):
    # 23-bit partial sums: |A|,|B| <= 4, outlier rows with a_s = 2^3, K = 4096
    M, N, K = 96, 256, 4096
    d = workloads.make_exact_inputs(M, N, K, seed=5, u_range=(-2, 0), v_range=(-2, 0),
                                    outlier_rows=[0, 33, 95], outlier_u=3)
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    dd = to_dev(d)
    for variant, S in (("generic", 0), ("swap_ab", 0), ("swap_ab_splitk", 4)):
        assert_bitwise(run(gpu, dd, "fp32", variant, S), ref, "fp32", variant)


def test_mfma_group_sum_is_exact_to_16_bits(gpu):
    # Same-sign group sums reaching 2^15 plus odd unit terms: exact only if the
    # FP8 MFMA keeps full precision inside one 128-wide group.
    M, N, K = 32, 64, 256
    rng = np.random.default_rng(3)
    Ai = np.full((M, K), 16, np.int64)
    Bi = np.full((N, K), 16, np.int64)
    Ai[:, ::2] = 1
    Bi[:, ::3] = rng.choice([1, 15], size=Bi[:, ::3].shape)
    d = {"A": workloads.e4m3_code_of_int(Ai), "B": workloads.e4m3_code_of_int(Bi),
         "a_s": np.ones((M, 2), np.float32), "b_s": np.ones((1, 2), np.float32)}
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    for variant in ("generic", "swap_ab", "short_k256"):
        assert_bitwise(run(gpu, to_dev(d), "fp32", variant), ref, "fp32", variant)


@pytest.mark.parametrize("variant", ["generic", "swap_ab", "short_k256", "swap_ab_splitk"])
def test_identity_weight_decodes_every_code(gpu, variant):
    K = N = 256
    non_nan = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = np.concatenate([non_nan, np.zeros(2, np.uint8)])
    rng = np.random.default_rng(1)
    A = np.stack([codes] + [rng.permutation(codes) for _ in range(20)]).astype(np.uint8)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), np.arange(K)] = 0x38
    a_s = np.exp2(rng.integers(-3, 3, size=(A.shape[0], 2))).astype(np.float32)
    d = {"A": A, "a_s": a_s, "B": B, "b_s": np.ones((2, 2), np.float32)}
    ref = oracle.block_gemm(A, a_s, B, d["b_s"])
    S = 2 if variant == "swap_ab_splitk" else 0
    for out in OUTS:
        assert_bitwise(run(gpu, to_dev(d), out, variant, S), ref, out, f"{variant} {out}")


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_handworked_cases_on_gpu(gpu, case):
    for out in OUTS:
        C = run(gpu, to_dev(case), out)
        assert_bitwise(C, case["C"], out, f"{case['name']} {out}")
        if case["C_bits"] and out in case["C_bits"]:
            assert int(bits(C, out)[0, 0]) == int(case["C_bits"][out], 16)


def test_split_k_one_equals_swap_ab_bitwise(gpu):
    d = workloads.make_inputs(64, 512, 2048, seed=12)
    dd = to_dev(d)
    for cfg in (0, 6, 7):
        a = run(gpu, dd, "bf16", "swap_ab", 0, cfg)
        b = run(gpu, dd, "bf16", "swap_ab_splitk", 1, cfg)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), cfg


def test_deterministic_runs_and_streams(gpu):
    d = workloads.make_inputs(64, 512, 4096, seed=2)
    dd = to_dev(d)
    for variant, S in (("swap_ab_splitk", 8), ("generic", 0), ("swap_ab", 0)):
        base = run(gpu, dd, "fp32", variant, S)
        for _ in range(3):
            assert torch.equal(base.view(torch.int32), run(gpu, dd, "fp32", variant, S).view(torch.int32))
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            other = run(gpu, dd, "fp32", variant, S, stream=s)
        assert torch.equal(base.view(torch.int32), other.view(torch.int32))


def test_concurrent_streams_with_library_workspace(gpu):
    d1 = workloads.make_inputs(64, 512, 4096, seed=21)
    d2 = workloads.make_inputs(32, 1024, 2048, seed=22)
    r1 = oracle.block_gemm(d1["A"], d1["a_s"], d1["B"], d1["b_s"])
    r2 = oracle.block_gemm(d2["A"], d2["a_s"], d2["B"], d2["b_s"])
    dd1, dd2 = to_dev(d1), to_dev(d2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            c1 = gpu.gemm(dd1["A"], dd1["a_s"], dd1["B"], dd1["b_s"], variant="swap_ab_splitk", split_k=8,
                          workspace="library")
        with torch.cuda.stream(s2):
            c2 = gpu.gemm(dd2["A"], dd2["a_s"], dd2["B"], dd2["b_s"], variant="swap_ab_splitk", split_k=4,
                          workspace="library")
        outs.append((c1, c2))
    torch.cuda.synchronize()
    for c1, c2 in outs:
        assert_within_tolerance(c1, r1, "bf16")
        assert_within_tolerance(c2, r2, "bf16")


def test_concurrent_streams_with_default_workspace(gpu):
    """The binding's default split-K workspace (a zeroed tensor from torch's
    allocator on the call's stream) on two streams at once."""
    d1 = workloads.make_inputs(32, 512, 16384, seed=23)
    d2 = workloads.make_inputs(16, 512, 16384, seed=24)
    r1 = oracle.block_gemm(d1["A"], d1["a_s"], d1["B"], d1["b_s"])
    r2 = oracle.block_gemm(d2["A"], d2["a_s"], d2["B"], d2["b_s"])
    dd1, dd2 = to_dev(d1), to_dev(d2)
    assert gpu.plan(32, 512, 16384)["split_k"] > 1 and gpu.plan(16, 512, 16384)["split_k"] > 1
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            c1 = gpu.gemm(dd1["A"], dd1["a_s"], dd1["B"], dd1["b_s"])
        with torch.cuda.stream(s2):
            c2 = gpu.gemm(dd2["A"], dd2["a_s"], dd2["B"], dd2["b_s"])
        outs.append((c1, c2))
    torch.cuda.synchronize()
    for c1, c2 in outs:
        assert_within_tolerance(c1, r1, "bf16")
        assert_within_tolerance(c2, r2, "bf16")


def test_caller_workspace_is_reused_and_left_zeroed(gpu):
    M, N, K, S = 64, 512, 4096, 8
    n = gpu.workspace_size(M, N, K, "swap_ab_splitk", S)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    for seed in (31, 32, 33):
        d = workloads.make_inputs(M, N, K, seed=seed)
        ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        C = run(gpu, to_dev(d), "bf16", "swap_ab_splitk", S, workspace=ws)
        assert_within_tolerance(C, ref, "bf16", f"seed {seed}")
    plan = gpu.plan(M, N, K, torch.bfloat16, torch.cuda.get_device_properties(0).multi_processor_count,
                    "swap_ab_splitk", S)
    tiles = -(-M // plan["tile_m"]) * -(-N // plan["tile_n"])
    counters = ws[n - 4 * tiles:].view(torch.int32)
    assert int(counters.abs().sum()) == 0


@pytest.mark.parametrize("variant", ["auto", "generic", "swap_ab", "short_k256", "swap_ab_splitk"])
def test_guard_bands_untouched(gpu, variant):
    M, N, K = 37, 261, 256
    d = workloads.make_inputs(M, N, K, seed=4)
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    pad = 1024
    for out in OUTS:
        dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[out]
        buf = torch.full((pad + M * N + pad,), 7.0, dtype=dt, device="cuda:0")
        C = buf[pad:pad + M * N].view(M, N)
        run(gpu, to_dev(d), out, variant, 2 if variant == "swap_ab_splitk" else 0, C=C)
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + M * N:] == 7.0), f"{variant} {out}"
        assert_within_tolerance(C, ref, out, f"{variant} {out}")


def test_empty_and_degenerate_shapes(gpu):
    dev = "cuda:0"
    f8 = torch.float8_e4m3fn
    # M == 0 and N == 0: success, nothing written
    for M, N in ((0, 256), (16, 0)):
        A = torch.zeros((M, 256), dtype=f8, device=dev)
        B = torch.zeros((N, 256), dtype=f8, device=dev)
        C = gpu.gemm(A, torch.ones((M, 2), device=dev), B, torch.ones(((N + 127) // 128, 2), device=dev))
        assert C.shape == (M, N)
    # K == 0: the empty sum
    C = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device=dev)
    gpu.gemm(torch.zeros((5, 0), dtype=f8, device=dev), torch.zeros((5, 0), device=dev),
             torch.zeros((7, 0), dtype=f8, device=dev), torch.zeros((1, 0), device=dev), out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 0) and not torch.any(torch.signbit(C.float()))
    # single element, single column, N not a multiple of 4
    for (M, N, K) in ((1, 1, 128), (3, 1, 256), (2, 5, 384), (1, 131, 1024)):
        d = workloads.make_inputs(M, N, K, seed=M + N + K)
        ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
        for variant in ("auto", "generic", "swap_ab", "swap_ab_splitk"):
            assert_within_tolerance(run(gpu, to_dev(d), "fp32", variant), ref, "fp32", f"{variant} {M},{N},{K}")


def test_error_statuses(gpu):
    d = to_dev(workloads.make_inputs(16, 256, 512, seed=1))
    with pytest.raises(gpu.FP8BGError) as e:
        gpu.gemm(d["A"], d["a_s"], d["B"], d["b_s"], variant="short_k256")
    assert e.value.status == gpu.UNSUPPORTED
    with pytest.raises(gpu.FP8BGError) as e:
        gpu.gemm(d["A"], d["a_s"], d["B"], d["b_s"], variant="swap_ab", split_k=2)
    assert e.value.status == gpu.UNSUPPORTED
    with pytest.raises(gpu.FP8BGError) as e:
        gpu.gemm(d["A"], d["a_s"], d["B"], d["b_s"], variant="swap_ab_splitk", split_k=5)
    assert e.value.status == gpu.UNSUPPORTED       # S > K/128
    with forced_config(23), pytest.raises(gpu.FP8BGError) as e:   # 8-row tiles never split
        gpu.gemm(d["A"], d["a_s"], d["B"], d["b_s"], variant="swap_ab_splitk", split_k=2)
    assert e.value.status == gpu.UNSUPPORTED
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(gpu.FP8BGError) as e:
        gpu.gemm(d["A"], d["a_s"], d["B"], d["b_s"], variant="swap_ab_splitk", split_k=4, workspace=ws)
    assert e.value.status == gpu.OUT_OF_MEMORY


@pytest.mark.parametrize("variant,split", [("generic", 0), ("swap_ab", 0), ("swap_ab_splitk", 2), ("short_k256", 0)])
def test_fp16_overflow_rounds_to_infinity(gpu, variant, split):
    """fp16 output at its overflow threshold: exact sums 65519 (-> 65504),
    65520 (the tie past the largest finite value -> +Inf), -65520 (-> -Inf)
    and 2.57e7 (-> +Inf), bit for bit against the oracle's one-step rounding;
    bf16 and fp32 of the same sums stay finite and exact."""
    K = 256
    codes = {v: int(workloads.e4m3_code_of_int(np.array([v]))[0]) for v in (1, 15, 16, 96, 448)}

    def row(values):
        r = np.zeros(K, dtype=np.uint8)
        for k, v in enumerate(values):
            r[k] = codes[abs(v)] | (0x80 if v < 0 else 0)
        return r

    B = np.stack([row([448] * 146 + [96, 15]),             # 65519
                  row([448] * 146 + [96, 16]),             # 65520
                  row([-448] * 146 + [-96, -16]),          # -65520
                  row([448] * 128)])                       # 57344 per activation unit
    A = np.zeros((3, K), dtype=np.uint8)
    A[0] = codes[1]                                        # all ones
    A[1] = codes[1]
    A[2, :128] = codes[448]                                # 448 * 57344 * ... -> 2.57e7 on column 3
    d = {"A": A, "a_s": np.ones((3, 2), np.float32), "B": B, "b_s": np.ones((1, 2), np.float32)}
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    assert ref[0, 0] == 65519 and ref[0, 1] == 65520 and ref[0, 2] == -65520 and ref[2, 3] == 448 * 448 * 128
    dd = to_dev(d)
    C = run(gpu, dd, "fp16", variant, split)
    got = bits(C, "fp16")
    want = oracle.round_bits(ref, "fp16")
    assert got[0, 0] == 0x7BFF and got[0, 1] == 0x7C00 and got[0, 2] == 0xFC00 and got[2, 3] == 0x7C00
    assert np.array_equal(got, want)
    for out in ("bf16", "fp32"):
        assert_bitwise(run(gpu, dd, out, variant, split), ref, out, f"{variant} {out}")
