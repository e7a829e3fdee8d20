"""Seeded synthetic inputs for the block-scaled FP8 GEMM.

Shared by the tests, the smoke check and the benchmark, on both sides of a
parity check (the oracle and the HIP path).  This module builds inputs only:
it holds none of the GEMM's arithmetic.

Recipe (shapes and value distributions of the workloads the pages measure:
FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for Hopper",
section "Performance", DeepSeek-V4-Flash trace shape sets
N in {512, 1536, 4096, 8192}, K in {256, 1024, 4096}, M in [1, 16384]):

  * activations X [M,K]: fp32 N(0,1) draws, rounded to bf16 (RNE), optionally
    with a seeded 1% of rows multiplied by 10 (outlier tokens);
    per 1x128 group amax -> a_s = max(amax, 1e-12) / 448 (fp32);
    codes = E4M3_RNE(clamp(x / a_s, -448, 448));
  * weights W [N,K]: fp32 N(0, sigma=0.02) draws rounded to bf16; per 128x128
    block amax -> b_s likewise; codes the same way;
  * the clamp is needed because torch's E4M3 cast does not saturate.

The "exact" recipe draws integer-valued E4M3 codes in [-r, r] and
power-of-two scales, so that every partial sum is exact in fp32 and the GPU
result must equal the oracle bit for bit.

Randomness: numpy ``default_rng(seed)`` (PCG64).  The same seed always gives
the same bytes.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

GROUP = 128
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    outlier_frac: float = 0.0
    out_dtypes: tuple = ("bf16",)
    sweep_M: tuple = field(default=())
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five shapes the pages' traces are drawn from, named by what they are.
WORKLOADS = {
    "small_16x512x256": Workload("small_16x512x256", 16, 512, 256, seed=1,
                                 note="small case, N=512 K=256"),
    "decode_64x512x4096": Workload("decode_64x512x4096", 64, 512, 4096, seed=2,
                                   note="decode, skinny long-K (printed row 1,64,512,4096)"),
    "shortk_184x4096x256": Workload("shortk_184x4096x256", 184, 4096, 256, seed=3,
                                    sweep_M=(1, 36, 100, 214, 264),
                                    note="short-K projection (printed row 1,184,4096,256)"),
    "midm_128x8192x1024": Workload("midm_128x8192x1024", 128, 8192, 1024, seed=4,
                                   sweep_M=(1, 16, 64, 128, 256, 512),
                                   note="mid-M wide, K=1024 band"),
    "prefill_16384x4096x4096": Workload("prefill_16384x4096x4096", 16384, 4096, 4096, seed=5,
                                        outlier_frac=0.01, out_dtypes=("bf16", "fp32"),
                                        note="prefill, compute-bound, 1% outlier tokens"),
}
ORDER = list(WORKLOADS)


def sweep_seed(w: Workload, M: int) -> int:
    # A reshaped workload ("name:N..:K..", the benchmark's tuning runs) draws
    # from its base workload's seeds.
    return 100 * (ORDER.index(w.name.split(":")[0]) + 1) + M


def groups(K: int) -> int:
    return (K + GROUP - 1) // GROUP


def _to_bf16_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float()


def _encode_e4m3(q: torch.Tensor) -> np.ndarray:
    q = torch.clamp(q, -E4M3_MAX, E4M3_MAX)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_rows(x: np.ndarray):
    """Per 1x128 group quantisation of [M,K] (K % 128 == 0) -> (codes, scales [M,G])."""
    t = _to_bf16_f32(x)
    M, K = t.shape
    G = groups(K)
    tg = t.view(M, G, GROUP)
    amax = tg.abs().amax(dim=2)
    s = torch.clamp(amax, min=1e-12) / E4M3_MAX
    codes = _encode_e4m3(tg / s.unsqueeze(2)).reshape(M, K)
    return codes, s.numpy().astype(np.float32)


def quantize_blocks(w: np.ndarray):
    """Per 128x128 block quantisation of [N,K] (K % 128 == 0) -> (codes, scales [NB,G])."""
    t = _to_bf16_f32(w)
    N, K = t.shape
    G = groups(K)
    NB = (N + GROUP - 1) // GROUP
    pad = NB * GROUP - N
    tp = torch.nn.functional.pad(t, (0, 0, 0, pad)) if pad else t
    tb = tp.view(NB, GROUP, G, GROUP)
    amax = tb.abs().amax(dim=(1, 3))
    s = torch.clamp(amax, min=1e-12) / E4M3_MAX
    q = tb / s.view(NB, 1, G, 1)
    codes = _encode_e4m3(q).reshape(NB * GROUP, K)[:N]
    return np.ascontiguousarray(codes), s.numpy().astype(np.float32)


def make_inputs(M: int, N: int, K: int, seed: int, outlier_frac: float = 0.0):
    """Standard recipe: dict(A, a_s, B, b_s, outliers) as numpy arrays
    (uint8 codes, float32 scales, int64 indices of the x10 outlier rows)."""
    if K % GROUP:
        raise ValueError("the recipe quantises whole 128-wide groups")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    mask = np.zeros(M, dtype=bool)
    if outlier_frac > 0.0 and M:
        mask = rng.random(M) < outlier_frac
        x[mask] *= 10.0
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    A, a_s = quantize_rows(x)
    B, b_s = quantize_blocks(w)
    return {"A": A, "a_s": a_s, "B": B, "b_s": b_s, "outliers": np.nonzero(mask)[0]}


def make_workload(w: Workload, M: int = None):
    """Inputs of a named workload, optionally at one of its sweep M values."""
    M = w.M if M is None else M
    seed = w.seed if M == w.M else sweep_seed(w, M)
    return make_inputs(M, w.N, w.K, seed, w.outlier_frac)


def e4m3_code_of_int(v: np.ndarray) -> np.ndarray:
    """E4M3 codes of small integers (|v| <= 16), through torch's exact cast."""
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy().copy()


def make_exact_inputs(M: int, N: int, K: int, seed: int, int_range: int = 4,
                      u_range=(-2, 1), v_range=(-2, 1), outlier_rows=None, outlier_u: int = 3):
    """Integer-valued E4M3 codes in [-int_range, int_range] and power-of-two scales
    a_s = 2^u, b_s = 2^v; optional rows whose a_s exponent is outlier_u.
    Returns dict(A, a_s, B, b_s, Ai, Bi, u, v) with the integer data alongside."""
    rng = np.random.default_rng(seed)
    G = groups(K)
    NB = (N + GROUP - 1) // GROUP
    Ai = rng.integers(-int_range, int_range + 1, size=(M, K), dtype=np.int64)
    Bi = rng.integers(-int_range, int_range + 1, size=(N, K), dtype=np.int64)
    u = rng.integers(u_range[0], u_range[1] + 1, size=(M, G), dtype=np.int64)
    v = rng.integers(v_range[0], v_range[1] + 1, size=(NB, G), dtype=np.int64)
    if outlier_rows is not None and len(outlier_rows):
        u[np.asarray(outlier_rows)] = outlier_u
    return {
        "A": e4m3_code_of_int(Ai), "B": e4m3_code_of_int(Bi),
        "a_s": np.ldexp(np.float32(1.0), u).astype(np.float32),
        "b_s": np.ldexp(np.float32(1.0), v).astype(np.float32),
        "Ai": Ai, "Bi": Bi, "u": u, "v": v,
    }


# ---------------------------------------------------------------------------
# Grouped (mixture-of-experts) inputs: tokens routed top-k over E experts,
# the routed rows grouped by expert, one weight [N,K] per expert.  Shapes of
# the MoE kernel page (section "Performance": the Flash shape's 256 experts,
# t16 .. t1024 tokens) with the first page's decode weight shape
# (N=512, K=4096); routing is uniform, each token picks top_k distinct
# experts.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class MoEWorkload:
    name: str
    tokens: int
    experts: int
    top_k: int
    N: int
    K: int
    seed: int
    note: str = ""


MOE_WORKLOADS = {
    "moe_decode_t64_e256_512x4096": MoEWorkload("moe_decode_t64_e256_512x4096", 64, 256, 8, 512, 4096, seed=11,
                                                note="MoE decode: 64 tokens, top-8 of 256 experts, expert weight 512x4096"),
    "moe_t16_e256_512x4096": MoEWorkload("moe_t16_e256_512x4096", 16, 256, 8, 512, 4096, seed=12,
                                         note="16 tokens: about half the experts hold a row"),
    "moe_t256_e256_512x4096": MoEWorkload("moe_t256_e256_512x4096", 256, 256, 8, 512, 4096, seed=13,
                                          note="256 tokens: 8 rows per expert on average"),
    "moe_t1024_e256_512x4096": MoEWorkload("moe_t1024_e256_512x4096", 1024, 256, 8, 512, 4096, seed=14,
                                           note="1024 tokens: 32 rows per expert on average"),
    "moe_t2048_e256_512x4096": MoEWorkload("moe_t2048_e256_512x4096", 2048, 256, 8, 512, 4096, seed=16,
                                           note="2048 tokens: 64 rows per expert on average"),
    "moe_t4096_e256_512x4096": MoEWorkload("moe_t4096_e256_512x4096", 4096, 256, 8, 512, 4096, seed=15,
                                           note="4096 tokens (prefill): 128 rows per expert on average"),
}


def route_counts(tokens: int, experts: int, top_k: int, seed: int) -> np.ndarray:
    """Rows per expert when each token picks top_k distinct experts uniformly."""
    rng = np.random.default_rng(seed)
    picks = np.argsort(rng.random((tokens, experts)), axis=1)[:, :top_k]
    return np.bincount(picks.ravel(), minlength=experts).astype(np.int64)


def offsets_of(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def make_grouped_inputs(counts, N: int, K: int, seed: int, chunk_experts: int = 16):
    """Standard recipe per expert: dict(A [M,K], a_s [M,G], B [E,N,K],
    b_s [E,ceil(N/128),G], offsets [E+1]) as numpy arrays.  The activations
    of the routed rows follow the activation recipe, every expert's weight the
    weight recipe (its own 128x128 blocks)."""
    if K % GROUP:
        raise ValueError("the recipe quantises whole 128-wide groups")
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    offsets = offsets_of(counts)
    M = int(offsets[-1])
    rng = np.random.default_rng(seed)
    A, a_s = quantize_rows(rng.standard_normal((M, K), dtype=np.float32))
    G, NB = groups(K), (N + GROUP - 1) // GROUP
    B = np.empty((E, N, K), dtype=np.uint8)
    b_s = np.empty((E, NB, G), dtype=np.float32)
    for e0 in range(0, E, chunk_experts):
        e1 = min(E, e0 + chunk_experts)
        w = rng.standard_normal((e1 - e0, N, K), dtype=np.float32) * np.float32(0.02)
        if N % GROUP == 0:      # blocks never straddle two experts: one call for the chunk
            q, s = quantize_blocks(w.reshape(-1, K))
            B[e0:e1] = q.reshape(e1 - e0, N, K)
            b_s[e0:e1] = s.reshape(e1 - e0, NB, G)
        else:
            for e in range(e0, e1):
                B[e], b_s[e] = quantize_blocks(w[e - e0])
    return {"A": A, "a_s": a_s, "B": B, "b_s": b_s, "offsets": offsets}


def make_moe_workload(w: MoEWorkload):
    counts = route_counts(w.tokens, w.experts, w.top_k, w.seed)
    return make_grouped_inputs(counts, w.N, w.K, w.seed + 1)


def make_exact_grouped_inputs(counts, N: int, K: int, seed: int, int_range: int = 4):
    """Integer-valued codes and power-of-two scales (as make_exact_inputs),
    per expert: every partial sum is exact in fp32."""
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    offsets = offsets_of(counts)
    M = int(offsets[-1])
    d = make_exact_inputs(M, N * E, K, seed, int_range=int_range)
    G, NB = groups(K), (N + GROUP - 1) // GROUP
    rng = np.random.default_rng(seed + 1)
    v = rng.integers(-2, 2, size=(E, NB, G))
    return {"A": d["A"], "a_s": d["a_s"], "B": d["B"].reshape(E, N, K),
            "b_s": np.ldexp(np.float32(1.0), v).astype(np.float32), "offsets": offsets}
