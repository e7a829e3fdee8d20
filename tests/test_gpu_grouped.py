"""GPU parity of the grouped (mixture-of-experts) block-scaled GEMM
(fp8_block_gemm_grouped, through the C ABI) with the CPU oracle.

Every tile configuration is forced on expert groups that include empty
experts, single-row experts and experts spanning several token tiles, with
ragged N tails, for each output dtype: within |dC| <= 2 ulp(|C_ref|) +
1e-3 rms(C_ref) on the standard recipe, bit for bit on integer-valued
inputs with power-of-two scales.  At the MoE decode size (64 tokens routed
top-8 over 256 experts, expert weights 512 x 4096), with the launch the
benchmark times, sampled rows are checked against the oracle.

MoE-style traffic: FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8
matmul for Hopper", section "Description"; per-expert token groups and the
decode swap-AB path: the MoE kernel page, section "Summary".
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_gemm_amd as fbg
import oracle
import workloads
from tests._gpu import TORCH_OUT, assert_bitwise, assert_within_tolerance, forced_config

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (forced config, rows per expert, N, K): every configuration, empty experts,
# experts of one row and experts spanning several token tiles, ragged N.
GROUPED_CASES = [
    (0, [3, 0, 17, 1, 40, 0, 9], 300, 1024),
    (0, [16, 16, 0, 33], 130, 4096),
    (1, [0, 5, 70, 2, 31], 515, 512),
    (1, [64], 200, 256),
    (2, [130, 0, 1, 65, 7], 260, 1024),
    (2, [0, 0, 200], 140, 384),
    (3, [9, 0, 20, 1], 300, 640),
    (3, [1] * 24, 130, 256),
    (4, [12, 50, 0, 3], 600, 1024),
    (4, [2, 2, 2], 257, 2048),
    (5, [3, 0, 17, 40], 300, 4096),
    (5, [100, 1], 130, 1152),
    (6, [3, 0, 17, 40, 64, 65, 130], 300, 4096),
    (6, [5, 1, 0, 33], 257, 1152),
    (7, [9, 0, 20, 1, 32, 33], 130, 2048),
    (7, [33, 2], 300, 640),
    (8, [12, 0, 3, 30, 48, 49], 515, 1024),
    (8, [1, 70], 140, 384),
    (9, [7, 0, 40, 64, 100], 600, 4096),
    (9, [2, 17, 50], 130, 1024),
    (10, [7, 0, 40, 31], 600, 2048),
    (10, [16, 17], 260, 1024),
]

# The generic kernel in grouped mode: configuration 11 + c runs generic tile
# configuration c (BM x BN: 0 128x128, 1 256x128, 2 64x128, 3 256x256,
# 4 64x64, 5 128x64, 6 64x32, 7 128x256).  Experts spanning several row tiles, empty
# experts, more than 64 experts (the tile scan's second chunk), ragged N.
GENERIC_GROUPED_CASES = [
    (11, [130, 0, 1, 300, 7], 300, 1024),
    (11, [3] * 70 + [200], 130, 256),
    (12, [513, 0, 40], 260, 512),
    (12, [1, 257, 256], 130, 384),
    (13, [65, 0, 64, 129, 3], 515, 1024),
    (13, [5] * 100, 200, 256),
    (14, [300, 1, 0, 257], 600, 640),
    (14, [256, 256], 257, 256),
    (14, [130, 0, 3, 257], 300, 3200),
    (15, [65, 0, 64, 129, 3], 300, 2048),
    (15, [1] * 130, 140, 256),
    (16, [129, 0, 128, 1, 200], 260, 1024),
    (16, [7, 0, 0, 300], 130, 384),
    (17, [65, 0, 64, 129, 3], 300, 1024),
    (17, [2] * 66, 130, 512),
    (18, [65, 0, 64, 129, 3], 515, 1024),
    (18, [130, 0, 3, 257], 300, 3200),
    (18, [2] * 70, 260, 256),
]
GROUPED_CASES = GROUPED_CASES + GENERIC_GROUPED_CASES


def to_dev(d):
    return {
        "A": torch.from_numpy(np.ascontiguousarray(d["A"])).to(DEV).view(torch.float8_e4m3fn),
        "a_s": torch.from_numpy(np.ascontiguousarray(d["a_s"])).to(DEV),
        "B": torch.from_numpy(np.ascontiguousarray(d["B"])).to(DEV).view(torch.float8_e4m3fn),
        "b_s": torch.from_numpy(np.ascontiguousarray(d["b_s"])).to(DEV),
        "offsets": torch.from_numpy(np.asarray(d["offsets"], dtype=np.int32)).to(DEV),
    }


def run(dd, out="bf16", cfg=None, C=None, stream=None):
    with forced_config(cfg):
        C = fbg.grouped_gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], dd["offsets"], out_dtype=TORCH_OUT[out],
                             out=C, stream=stream)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("out", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("cfg,counts,N,K", GROUPED_CASES)
def test_grouped_configs_within_tolerance(gpu, cfg, counts, N, K, out):
    d = workloads.make_grouped_inputs(counts, N, K, seed=cfg * 100 + N + K)
    ref = oracle.grouped_gemm(d["A"], d["a_s"], d["B"], d["b_s"], d["offsets"])
    C = run(to_dev(d), out, cfg)
    assert_within_tolerance(C, ref, out, f"grouped cfg {cfg} counts {counts} N={N} K={K} {out}")


@pytest.mark.parametrize("cfg,counts,N,K", GROUPED_CASES)
def test_grouped_configs_bitwise_exact_mode(gpu, cfg, counts, N, K):
    d = workloads.make_exact_grouped_inputs(counts, N, K, seed=7 + cfg)
    ref = oracle.grouped_gemm(d["A"], d["a_s"], d["B"], d["b_s"], d["offsets"])
    for out in ("fp32", "bf16"):
        C = run(to_dev(d), out, cfg)
        assert_bitwise(C, ref, out, f"grouped exact cfg {cfg} {out}")


@pytest.mark.parametrize("E", [1, 3, 8, 64])
def test_grouped_auto_config(gpu, E):
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 24, E)
    if E > 1:
        counts[rng.integers(0, E)] = 0
    d = workloads.make_grouped_inputs(counts, 260, 1024, seed=E)
    ref = oracle.grouped_gemm(d["A"], d["a_s"], d["B"], d["b_s"], d["offsets"])
    C = run(to_dev(d))
    assert_within_tolerance(C, ref, "bf16", f"grouped auto E={E}")


def test_single_expert_equals_plain_gemm_bitwise_in_exact_mode(gpu):
    d = workloads.make_exact_grouped_inputs([77], 300, 1024, seed=3)
    dd = to_dev(d)
    C1 = run(dd, "fp32")
    C2 = fbg.gemm(dd["A"], dd["a_s"], dd["B"][0], dd["b_s"][0], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    assert_bitwise(C1, oracle.block_gemm(d["A"], d["a_s"], d["B"][0], d["b_s"][0]), "fp32", "E=1")


def test_moe_decode_size_sampled_rows(gpu):
    """The MoE decode workload at full size with the auto launch: 64 sampled
    rows (each against the oracle's GEMM of the row's own expert), and two
    calls give the same bits."""
    w = workloads.MOE_WORKLOADS["moe_decode_t64_e256_512x4096"]
    d = workloads.make_moe_workload(w)
    dd = to_dev(d)
    C = run(dd)
    C2 = run(dd)
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    off = d["offsets"]
    M = int(off[-1])
    rows = np.unique(np.concatenate([np.random.default_rng(0).choice(M, 62, replace=False), [0, M - 1]]))
    got = C.float().cpu().double().numpy()
    for m in rows:
        e = int(np.searchsorted(off, m, side="right") - 1)
        ref = oracle.block_gemm(d["A"][m:m + 1], d["a_s"][m:m + 1], d["B"][e], d["b_s"][e])
        tol = oracle.tolerance(ref, "bf16")
        assert np.all(np.abs(got[m:m + 1] - ref) <= tol), f"row {m} (expert {e})"


@pytest.mark.parametrize("cfg", [None, 11, 14])
def test_rows_outside_every_expert_are_untouched_and_offsets_are_clamped(gpu, cfg):
    """Offsets are device data the kernel clamps into [0, M]: rows no expert
    holds keep the caller's values, offsets past M are cut at M, decreasing
    pairs are empty."""
    d = workloads.make_grouped_inputs([4, 6, 3], 130, 256, seed=5)
    dd = to_dev(d)
    M, N = 13, 130
    sentinel = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    # expert 0 holds rows [0,4); expert 1's pair decreases (4 -> 2) and
    # expert 2's is empty (2 -> 2): rows 4.. are held by no expert
    dd["offsets"] = torch.tensor([0, 4, 2, 2], dtype=torch.int32, device=DEV)
    C = run(dd, "fp32", cfg, C=sentinel.clone())
    ref = oracle.block_gemm(d["A"][0:4], d["a_s"][0:4], d["B"][0], d["b_s"][0])
    assert_within_tolerance(C[:4], ref, "fp32", "held rows")
    assert torch.equal(C[4:], sentinel[4:])
    # the last offset past M: the last expert's rows end at M
    dd["offsets"] = torch.tensor([0, 4, 10, 1000], dtype=torch.int32, device=DEV)
    C = run(dd, "fp32", cfg, C=sentinel.clone())
    ref = np.empty((M, N))
    for e, (r0, r1) in enumerate([(0, 4), (4, 10), (10, 13)]):
        ref[r0:r1] = oracle.block_gemm(d["A"][r0:r1], d["a_s"][r0:r1], d["B"][e], d["b_s"][e])
    assert_within_tolerance(C, ref, "fp32", "clamped offsets")


def test_degenerate_sizes(gpu):
    d = workloads.make_grouped_inputs([3, 2], 130, 256, seed=6)
    dd = to_dev(d)
    # K == 0: the empty sum
    C = fbg.grouped_gemm(dd["A"][:, :0], dd["a_s"][:, :0], dd["B"][:, :, :0], dd["b_s"][:, :, :0],
                         dd["offsets"], out=torch.full((5, 130), 3.0, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), torch.zeros_like(C).view(torch.int16))
    # E == 0: no expert holds a row -> zeros
    e0 = fbg.grouped_gemm(dd["A"], dd["a_s"], dd["B"][:0], dd["b_s"][:0], dd["offsets"][:1],
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(e0) == 0
    # M == 0 and N == 0: nothing launched
    z = torch.zeros(3, dtype=torch.int32, device=DEV)
    assert fbg.grouped_gemm(dd["A"][:0], dd["a_s"][:0], dd["B"], dd["b_s"], z).shape == (0, 130)
    assert fbg.grouped_gemm(dd["A"], dd["a_s"], dd["B"][:, :0], dd["b_s"][:, :0], dd["offsets"]).shape == (5, 0)
    with pytest.raises(fbg.FP8BGError) as e:
        with forced_config(99):
            fbg.grouped_gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], dd["offsets"])
    assert e.value.status == fbg.UNSUPPORTED


def test_side_stream_and_unaligned_output(gpu):
    """A caller's stream, and N % 4 != 0 (scalar stores on the tail)."""
    d = workloads.make_grouped_inputs([5, 0, 11], 130, 512, seed=8)
    ref = oracle.grouped_gemm(d["A"], d["a_s"], d["B"], d["b_s"], d["offsets"])
    dd = to_dev(d)
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        C = run(dd, "fp16", stream=s)
    assert_within_tolerance(C, ref, "fp16", "side stream")
    big = torch.empty(16 * 131 + 1, dtype=torch.bfloat16, device=DEV)
    Cv = big[1:1 + 16 * 130].view(16, 130)          # 2-byte aligned only
    C = run(dd, "bf16", C=Cv)
    assert_within_tolerance(C, ref, "bf16", "unaligned C")


def test_quantised_operands_feed_the_grouped_gemm(gpu):
    """End to end on the GPU: bf16 activations and per-expert bf16 weights
    quantised by the library's kernels, then the grouped GEMM; the codes and
    scales equal the oracle's bit for bit, so the GEMM equals the grouped
    GEMM on the oracle-quantised operands bit for bit, and the oracle's
    grouped GEMM on them within tolerance."""
    counts = [5, 0, 33, 2, 70]
    E, N, K = len(counts), 260, 1024
    off = np.concatenate([[0], np.cumsum(counts)])
    M = int(off[-1])
    rng = np.random.default_rng(77)
    to_bits = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    xb = to_bits(rng.normal(size=(M, K)))
    wb = to_bits(rng.normal(size=(E, N, K)) * 0.02)
    x = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    w = torch.from_numpy(wb.view(np.int16)).to(DEV).view(torch.bfloat16)
    A, a_s = fbg.quantize_rows(x)
    Bq = torch.empty((E, N, K), dtype=torch.float8_e4m3fn, device=DEV)
    b_s = torch.empty((E, (N + 127) // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(E):
        fbg.quantize_blocks(w[e], Bq[e], b_s[e])
    offsets = torch.from_numpy(off.astype(np.int32)).to(DEV)
    C = fbg.grouped_gemm(A, a_s, Bq, b_s, offsets)
    torch.cuda.synchronize()
    qa, sa = oracle.quantize_rows(xb)
    qb = np.empty((E, N, K), np.uint8)
    sb = np.empty((E, (N + 127) // 128, K // 128), np.float32)
    for e in range(E):
        qb[e], sb[e] = oracle.quantize_blocks(wb[e])
    assert np.array_equal(A.view(torch.uint8).cpu().numpy(), qa)
    assert np.array_equal(Bq.view(torch.uint8).cpu().numpy(), qb)
    dd = to_dev({"A": qa, "a_s": sa, "B": qb, "b_s": sb, "offsets": off})
    C2 = fbg.grouped_gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], dd["offsets"])
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    assert_within_tolerance(C, oracle.grouped_gemm(qa, sa, qb, sb, off), "bf16", "quantised grouped")
