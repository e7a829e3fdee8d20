"""GPU parity at the workloads' full sizes, through the dispatcher (the launch
configuration the benchmark times).

Shapes drawn from the pages' trace shape sets (FlagGems-vllm PR #693, "feat:
optimize w8a8 block fp8 matmul for Hopper", section "Performance"): the
small, decode, short-K and mid-M shapes are compared with the oracle on every
element (at sweep points with M >= 256 on every 8th row and the last row);
the 16384-row prefill shape on all outlier rows plus every 16th row at an
offset that walks the 16 rows of an MFMA block (16j + j mod 16), and on
every row and column through sums that hold at any size:
  sum_n C[m,n] = sum_g a_s[m,g] sum_{k in g} A[m,k] w_g[k],  w_g[k] = sum_n b_s[n/128,g] B[n,k]
  sum_m C[m,n] = sum_g b_s[n/128,g] sum_{k in g} B[n,k] v_g[k], v_g[k] = sum_m a_s[m,g] A[m,k]
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._cases import torch_decode
from tests._gpu import TORCH_OUT, as_f64, assert_within_tolerance, run, to_dev

pytestmark = pytest.mark.gpu


def _rows_sample(M, every):
    rows = np.arange(0, M, every)
    return np.unique(np.append(rows, M - 1))


def _lane_rows(M):
    """Every 16th row, offset so the sample walks all 16 rows of a 16-row MFMA
    block (row 16j + j mod 16), plus the last row."""
    j = np.arange(M // 16)
    return np.unique(np.append(16 * j + j % 16, M - 1))


def _check_rows(C, d, rows, out):
    ref = oracle.block_gemm(d["A"][rows], d["a_s"][rows], d["B"], d["b_s"])
    assert_within_tolerance(C[torch.from_numpy(rows).to(C.device)], ref, out, f"rows {rows[:4]}...")


@pytest.mark.parametrize("name", ["small_16x512x256", "decode_64x512x4096", "shortk_184x4096x256",
                                  "midm_128x8192x1024"])
def test_workload_full(gpu, name):
    w = W.WORKLOADS[name]
    d = W.make_workload(w)
    ref = oracle.block_gemm(d["A"], d["a_s"], d["B"], d["b_s"])
    dd = to_dev(d)
    for out in w.out_dtypes + ("fp32",):
        C = run(gpu, dd, out)
        assert_within_tolerance(C, ref, out, f"{name} {out}")


@pytest.mark.parametrize("name,M", [(n, m) for n in ("shortk_184x4096x256", "midm_128x8192x1024")
                                    for m in W.WORKLOADS[n].sweep_M])
def test_workload_sweep(gpu, name, M):
    w = W.WORKLOADS[name]
    d = W.make_workload(w, M)
    C = run(gpu, to_dev(d), "bf16")
    rows = _rows_sample(M, 8) if M >= 256 else np.arange(M)
    _check_rows(C, d, rows, "bf16")


@pytest.mark.parametrize("M,N,K,variant,cfg", [
    (16, 512, 256, "swap_ab", 2),         # K = 256, a 16x16 grid of at most one workgroup per CU
    (32, 1536, 256, "swap_ab", 2),
    (32, 8192, 256, "short_k256", 12),    # 16x16 short-K tiles, four workgroups per CU
    (256, 1536, 256, "short_k256", 13),   # 32x16 short-K tiles, three per CU
    (4096, 1536, 1024, "generic", 7),     # 128x256 where it ties with 256x128
    (1024, 8192, 1024, "generic", 7),
])
def test_dispatch_choice_at_sweep_shape(gpu, M, N, K, variant, cfg):
    """The automatic plan at shapes of the dispatch sweep where the rules pick
    these tiles, through fp8_block_gemm, against the oracle on every row for
    small M and on sampled lane rows otherwise."""
    p = gpu.plan(M, N, K)
    assert (p["variant_name"], p["config"]) == (variant, cfg)
    d = W.make_inputs(M, N, K, seed=71)
    C = run(gpu, to_dev(d), "bf16")
    rows = np.arange(M) if M <= 256 else _lane_rows(M)
    _check_rows(C, d, rows, "bf16")


def _row_col_sums(d):
    """fp64 row and column sums of C from O(MK + NK) work (see module doc)."""
    A, B = torch_decode(d["A"]), torch_decode(d["B"])
    M, K = A.shape
    N = B.shape[0]
    as_full = np.repeat(d["a_s"].astype(np.float64), 128, axis=1)
    bs_rows = np.repeat(d["b_s"].astype(np.float64), 128, axis=0)[:N]
    bs_full = np.repeat(bs_rows, 128, axis=1)
    Aw = A * as_full
    Bw = B * bs_full
    w = Bw.sum(axis=0)           # [K]
    v = Aw.sum(axis=0)           # [K]
    return Aw @ w, Bw @ v


def test_prefill_workload(gpu):
    w = W.WORKLOADS["prefill_16384x4096x4096"]
    d = W.make_workload(w)
    dd = to_dev(d)
    rows = np.unique(np.concatenate([d["outliers"], _lane_rows(w.M)]))
    rsum, csum = _row_col_sums(d)
    for out in w.out_dtypes:
        C = run(gpu, dd, out)
        _check_rows(C, d, rows, out)
        # Every row and column through sums: if each element meets
        # |dC| <= 2 ulp(|C_ref|) + 1e-3 rms(C_ref), a sum of elements is within
        # the sum of those bounds (ulp(|C_ref|) <= 2 ulp(|C|) here).
        Cd = C.double()
        rms = float(Cd.square().mean().sqrt())
        tol = torch.from_numpy(oracle.ulp(as_f64(C), out)).to(C.device) * 4 + 1e-3 * rms
        g_r, g_c = Cd.sum(dim=1).cpu().numpy(), Cd.sum(dim=0).cpu().numpy()
        b_r, b_c = tol.sum(dim=1).cpu().numpy(), tol.sum(dim=0).cpu().numpy()
        assert np.all(np.abs(g_r - rsum) <= b_r), f"row sums {out}"
        assert np.all(np.abs(g_c - csum) <= b_c), f"column sums {out}"
        del C, Cd, tol
        torch.cuda.empty_cache()


def test_prefill_shape_exact_mode(gpu):
    """Integer-valued inputs at the full prefill shape: sampled rows bit for
    bit against the oracle, and every row and column sum exactly equal to
    int64 arithmetic (C is exact in fp32, its fp64 sums are exact)."""
    M, N, K = 16384, 4096, 4096
    rng = np.random.default_rng(55)
    out_rows = np.sort(rng.choice(M, 160, replace=False))
    d = W.make_exact_inputs(M, N, K, seed=55, u_range=(-2, 0), v_range=(-2, 0), outlier_rows=out_rows)
    C = run(gpu, to_dev(d), "fp32")
    rows = np.unique(np.concatenate([out_rows, _lane_rows(M)]))
    ref = oracle.block_gemm(d["A"][rows], d["a_s"][rows], d["B"], d["b_s"])
    got = C[torch.from_numpy(rows).to(C.device)].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.round_bits(ref, "fp32"))
    # exact sums, scaled by 2^4 (u, v >= -2) to stay in integers
    Ai, Bi, u, v = d["Ai"], d["Bi"], d["u"], d["v"]
    G = K // 128
    nb = np.arange(N) // 128
    row16 = np.zeros(M, np.int64)
    col16 = np.zeros(N, np.int64)
    for g in range(G):
        ks = slice(128 * g, 128 * g + 128)
        wB = (Bi[:, ks] << (v[nb, g] + 2)[:, None]).sum(axis=0)          # [128]
        wA = (Ai[:, ks] << (u[:, g] + 2)[:, None]).sum(axis=0)           # [128]
        row16 += (Ai[:, ks] @ wB) << (u[:, g] + 2)
        col16 += (Bi[:, ks] @ wA) << (v[nb, g] + 2)
    Cd = C.double()
    assert np.array_equal(Cd.sum(dim=1).cpu().numpy() * 16, row16.astype(np.float64))
    assert np.array_equal(Cd.sum(dim=0).cpu().numpy() * 16, col16.astype(np.float64))
