"""The C-ABI boundary without a GPU: the library loads and exports every
function include/fp8bg.h declares; the dispatcher's plan (pure host code) and
the host-side argument validation return the documented decisions and
statuses.  No compute call is made (validation fails, or the shape is empty,
before any HIP call).

Dispatch contract (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8
matmul for Hopper", sections "Description" and "Numerical safety"): each
shape is routed by (M, N, K); each special path runs only under its guard;
every other shape falls through to the generic kernel.
"""
import ctypes
import os
import re

import pytest
import torch

import block_scaled_fp8_gemm_amd as fbg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bg.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp8_block_gemm\w*)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = fbg.load()
    names = declared_functions()
    assert len(names) >= 6, names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fp8_block_gemm_version() == 100


def test_status_strings():
    for st in range(6):
        assert len(fbg.status_string(st)) > 3
    assert fbg.status_string(99) == "unknown status"


def test_plan_for_the_workloads():
    # the small case: the swap-AB 16x16 tile (its grid of 32 fits one per CU)
    p = fbg.plan(16, 512, 256)
    assert (p["variant_name"], p["config"], p["split_k"], p["grid"]) == ("swap_ab", 2, 1, 32)
    # decode: the single-stage tile of 8 activation rows, unsplit, one
    # workgroup per CU
    p = fbg.plan(64, 512, 4096)
    assert (p["variant_name"], p["config"], p["split_k"], p["grid"]) == ("swap_ab", 23, 1, 256)
    assert fbg.plan(16, 512, 4096)["config"] == 23 and fbg.plan(16, 512, 4096)["split_k"] == 1
    # past one workgroup per CU in 8-row tiles, the 16x16 single-stage tile
    p = fbg.plan(128, 512, 4096)
    assert (p["config"], p["split_k"], p["grid"]) == (22, 1, 256)
    # K = 8192 with a grid of at most a quarter of the device splits K (with
    # a workspace), else the 8-row tile
    p = fbg.plan(16, 512, 8192)
    assert p["variant_name"] == "swap_ab_splitk" and p["split_k"] > 1 and p["workspace_bytes"] > 0
    assert fbg.plan(16, 512, 8192, split_k=1)["config"] == 23
    assert fbg.plan(64, 512, 8192)["config"] == 23
    # past 64 groups the split rule alone (a grid of at most three quarters of
    # the device)
    p = fbg.plan(32, 512, 16384)
    assert p["variant_name"] == "swap_ab_splitk" and p["split_k"] == 4
    # K = 256: the swap-AB 16x16 tile while its grid is at most one workgroup
    # per CU (M > 1), then short-K while its 16x16 grid fits four workgroups
    # per CU or its 32x16 grid three, the generic kernel beyond (measured
    # faster there)
    for M, N in ((2, 512), (128, 512), (32, 1536), (16, 4096)):
        p = fbg.plan(M, N, 256)
        assert (p["variant_name"], p["config"], p["split_k"]) == ("swap_ab", 2, 1), (M, N)
        grid = -(-N // 16) * -(-M // 16)
        assert fbg.plan(M, N, 256, cu_count=128)["variant_name"] == ("swap_ab" if grid <= 128 else "short_k256")
    assert fbg.plan(1, 512, 256)["variant_name"] == "swap_ab"      # one token: only up to 512 columns
    assert fbg.plan(1, 1536, 256)["variant_name"] == "short_k256"
    assert fbg.plan(17, 4096, 256)["variant_name"] == "short_k256"
    assert fbg.plan(32, 4096, 256)["variant_name"] == "short_k256"
    assert fbg.plan(128, 1536, 256)["variant_name"] == "short_k256"
    p = fbg.plan(32, 8192, 256)
    assert (p["variant_name"], p["config"]) == ("short_k256", 12)
    p = fbg.plan(256, 1536, 256)
    assert (p["variant_name"], p["config"]) == ("short_k256", 13)
    for M in (100, 184, 214, 264):
        assert fbg.plan(M, 4096, 256)["variant_name"] == "generic"
    assert fbg.plan(1024, 512, 256)["variant_name"] == "generic"
    # the 128x256 tile (8 waves) where it ties with 256x128 (4 waves)
    assert fbg.plan(4096, 1536, 1024)["config"] == 7
    assert fbg.plan(1024, 8192, 4096)["config"] == 7
    p = fbg.plan(128, 8192, 1024)
    assert p["variant_name"] in ("swap_ab", "swap_ab_splitk", "generic")
    # split-K only for long K with a grid of at most half the device
    assert fbg.plan(1, 512, 1024)["split_k"] == 1 and fbg.plan(64, 512, 1024)["split_k"] == 1
    assert fbg.plan(256, 512, 4096)["variant_name"] == "swap_ab"
    # swap-AB tiles (their fragments staged through LDS) up to three 16x16 or
    # two 32x16 workgroups per CU, the generic kernel past that (the measured
    # dispatch sweep); decode splits K for two workgroups per CU, at most 4
    p = fbg.plan(16, 512, 16384)
    assert (p["config"], p["split_k"]) == (2, 4)
    assert fbg.plan(64, 512, 1536)["config"] == 23 and fbg.plan(64, 512, 1024)["config"] != 23
    assert fbg.plan(1, 4096, 4096)["config"] == 11 and fbg.plan(1, 512, 4096)["config"] == 23
    assert fbg.plan(4, 1536, 4096)["config"] == 23 and fbg.plan(4, 4096, 4096)["config"] == 11
    assert fbg.plan(128, 512, 1024)["config"] == 2
    p = fbg.plan(512, 512, 4096)
    assert p["variant_name"] == "swap_ab" and p["config"] == 7
    assert fbg.plan(128, 1536, 4096)["variant_name"] == "swap_ab"
    assert fbg.plan(256, 1536, 4096)["variant_name"] == "generic"
    assert fbg.plan(64, 8192, 4096)["variant_name"] == "generic"
    p = fbg.plan(16384, 4096, 4096)
    assert p["variant_name"] == "generic" and p["workspace_bytes"] == 0 and p["config"] == 8
    assert (p["tile_m"], p["tile_n"], p["grid"]) == (256, 256, 1024)


@pytest.mark.parametrize("cu", [1, 8, 80, 256, 304, 1024])
def test_plan_is_consistent_for_any_cu_count(cu):
    for (M, N, K) in [(1, 4096, 1024), (64, 512, 4096), (300, 1000, 768), (16384, 4096, 4096), (7, 9, 128)]:
        p = fbg.plan(M, N, K, cu_count=cu)
        tiles = -(-M // p["tile_m"]) * -(-N // p["tile_n"])
        assert p["grid"] == tiles * p["split_k"]
        assert 1 <= p["split_k"] <= K // 128
        if p["split_k"] > 1:
            assert p["variant_name"] == "swap_ab_splitk"
            assert p["workspace_bytes"] >= p["split_k"] * tiles * p["tile_m"] * p["tile_n"] * 4 + 4 * tiles
        else:
            assert p["workspace_bytes"] == 0


def test_guard_fall_through_to_generic():
    # outside every special guard (K != 256, M large): generic
    for (M, N, K) in [(1025, 4096, 256), (300, 4096, 512), (5000, 300, 1152)]:
        assert fbg.plan(M, N, K)["variant_name"] == "generic"


def test_forced_variant_guards():
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(64, 512, 512, variant="short_k256")
    assert e.value.status == fbg.UNSUPPORTED
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(64, 512, 512, variant="swap_ab", split_k=2)
    assert e.value.status == fbg.UNSUPPORTED
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(64, 512, 512, variant="swap_ab_splitk", split_k=5)
    assert e.value.status == fbg.UNSUPPORTED
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(64, 512, 200)
    assert e.value.status == fbg.UNSUPPORTED
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(-1, 512, 256)
    assert e.value.status == fbg.INVALID_VALUE
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.plan(1, 512, 256, out_dtype=7)
    assert e.value.status == fbg.INVALID_VALUE
    p = fbg.plan(64, 512, 512, variant="swap_ab_splitk", split_k=1)
    assert p["split_k"] == 1 and p["workspace_bytes"] == 0
    assert fbg.plan(64, 512, 512, variant="generic")["variant_name"] == "generic"


def test_automatic_plan_without_a_split():
    # split_k = 1 under AUTO: the dispatcher's variant and tile with no K
    # split -- the plan fp8_block_gemm (no caller workspace) runs, so that
    # call never needs a workspace
    for (M, N, K) in [(64, 512, 4096), (16, 1536, 4096), (32, 512, 4096), (1, 512, 256), (16384, 4096, 4096),
                      (128, 8192, 1024), (300, 128, 2048)]:
        p = fbg.plan(M, N, K, variant="auto", split_k=1)
        assert p["split_k"] == 1 and p["workspace_bytes"] == 0, (M, N, K)
        assert p["variant_name"] != "swap_ab_splitk"
        q = fbg.plan(M, N, K)
        if q["split_k"] == 1:
            assert (p["variant_name"], p["config"]) == (q["variant_name"], q["config"]), (M, N, K)


def test_workspace_size_for_forced_split():
    n = fbg.workspace_size(64, 512, 4096, "swap_ab_splitk", 8)
    p = fbg.plan(64, 512, 4096, variant="swap_ab_splitk", split_k=8)
    assert n == p["workspace_bytes"] > 0
    assert fbg.workspace_size(64, 512, 4096, "generic", 1) == 0


def test_eight_row_tiles_never_split(monkeypatch):
    """The swap-AB tile of 8 activation rows (configuration 23) keeps its
    partials in 16-row blocks, so the planner refuses to split it over K."""
    monkeypatch.setenv("FBG_FORCE_CONFIG", "23")
    with pytest.raises(fbg.FP8BGError):
        fbg.workspace_size(64, 512, 4096, "swap_ab_splitk", 2)
    assert fbg.workspace_size(64, 512, 4096, "swap_ab", 1) == 0


def _call(A=0x10000, a_s=0x20000, B=0x30000, b_s=0x40000, C=0x50000000, M=16, N=256, K=256, out=0,
          variant=0, split=0, ws=None, wsn=0):
    lib = fbg.load()
    return lib.fp8_block_gemm_ex(A, a_s, B, b_s, C, M, N, K, out, None, variant, split, ws, wsn)


def test_host_validation_statuses():
    # Pointers are never dereferenced here: validation fails (or the shape is
    # empty) before any HIP call.
    assert _call(A=None) == fbg.INVALID_VALUE
    assert _call(a_s=None) == fbg.INVALID_VALUE
    assert _call(B=None) == fbg.INVALID_VALUE
    assert _call(b_s=None) == fbg.INVALID_VALUE
    assert _call(C=None) == fbg.INVALID_VALUE
    assert _call(M=-1) == fbg.INVALID_VALUE
    assert _call(out=3) == fbg.INVALID_VALUE
    assert _call(K=200) == fbg.UNSUPPORTED
    assert _call(K=(1 << 24) + 128) == fbg.UNSUPPORTED      # past the kernels' 32-bit row offsets
    assert _call(K=1 << 24) == fbg.UNSUPPORTED              # a 256-row tile would end at 2^32 bytes
    assert _call(A=0x10008) == fbg.UNSUPPORTED              # A not 16-byte aligned
    assert _call(B=0x30004) == fbg.UNSUPPORTED
    assert _call(a_s=0x20002) == fbg.UNSUPPORTED
    assert _call(C=0x50000001) == fbg.UNSUPPORTED           # bf16 C must be 2-byte aligned
    assert _call(C=0x10000 + 64) == fbg.INVALID_VALUE       # C overlaps A
    assert _call(C=0x40000) == fbg.INVALID_VALUE            # C overlaps b_s
    assert _call(M=0, A=None, a_s=None, C=None) == fbg.SUCCESS   # empty: nothing launched
    assert _call(N=0, B=None, b_s=None, C=None) == fbg.SUCCESS
    assert _call(variant=9) == fbg.INVALID_VALUE
    assert _call(split=-2) == fbg.INVALID_VALUE


def test_python_wrapper_checks():
    A = torch.zeros((4, 256), dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError):
        fbg.gemm(A, torch.zeros((4, 3)), torch.zeros((8, 256), dtype=torch.float8_e4m3fn), torch.zeros((1, 2)))
    with pytest.raises(TypeError):
        fbg.gemm(A.float(), torch.zeros((4, 2)), torch.zeros((8, 256), dtype=torch.float8_e4m3fn),
                 torch.zeros((1, 2)))
    with pytest.raises(ValueError):
        fbg.gemm(A, torch.zeros((4, 2)), torch.zeros((8, 256), dtype=torch.float8_e4m3fn)[:, ::1].t(),
                 torch.zeros((1, 2)))


def test_every_tile_configuration_has_parity_cases():
    """Every configuration the kernels can be launched with (the X-macro lists
    of csrc/fp8bg_configs.h) is forced by at least one GPU tolerance case."""
    text = open(os.path.join(ROOT, "block_scaled_fp8_gemm_amd", "csrc", "fp8bg_configs.h")).read()

    def ids(macro):
        body = re.search(r"#define %s\(X\)(.*?)\n\n" % macro, text, re.S).group(1)
        return {int(i) for i in re.findall(r"X\((\d+),", body)}

    from tests.test_gpu_parity import TOL_CASES
    have = {}
    for variant, cfg, *_ in TOL_CASES:
        family = "swap_ab" if variant.startswith("swap_ab") else variant
        have.setdefault(family, set()).add(cfg)
    assert ids("FBG_GENERIC_CFGS") <= have["generic"]
    assert ids("FBG_SWAP_CFGS") <= have["swap_ab"]
    assert ids("FBG_SHORT_CFGS") <= have["short_k256"]
    from tests.test_gpu_grouped import GROUPED_CASES
    grouped = {c[0] for c in GROUPED_CASES}
    n_skinny = len(ids("FBG_GROUPED_CFGS"))
    assert ids("FBG_GROUPED_CFGS") <= grouped
    # the generic kernel in grouped mode: configurations 0-7 (8 is dense-only)
    assert {n_skinny + c for c in ids("FBG_GENERIC_CFGS") if c < 8} <= grouped


def _qcall(x=0x100000, M=4, K=256, A=0x200000, a_s=0x300000):
    return fbg.load().fp8_block_gemm_quantize_rows(x, M, K, A, a_s, None)


def test_quantize_host_validation_statuses():
    # As above: every case fails validation (or is empty) before any HIP call.
    assert _qcall(x=None) == fbg.INVALID_VALUE
    assert _qcall(A=None) == fbg.INVALID_VALUE
    assert _qcall(a_s=None) == fbg.INVALID_VALUE
    assert _qcall(M=-1) == fbg.INVALID_VALUE
    assert _qcall(K=-128) == fbg.INVALID_VALUE
    assert _qcall(K=200) == fbg.UNSUPPORTED
    assert _qcall(x=0x100008) == fbg.UNSUPPORTED           # x not 16-byte aligned
    assert _qcall(A=0x200004) == fbg.UNSUPPORTED           # A not 8-byte aligned
    assert _qcall(a_s=0x300002) == fbg.UNSUPPORTED
    assert _qcall(A=0x100000 + 512) == fbg.INVALID_VALUE   # A overlaps x (x is 4*256*2 bytes)
    assert _qcall(a_s=0x200000 + 8) == fbg.INVALID_VALUE   # a_s overlaps A
    assert _qcall(M=0, x=None, A=None, a_s=None) == fbg.SUCCESS
    assert _qcall(K=0, x=None, A=None, a_s=None) == fbg.SUCCESS


def test_quantize_wrapper_checks():
    with pytest.raises(ValueError):
        fbg.quantize_rows(torch.zeros(4, 128, dtype=torch.float32))
    with pytest.raises(ValueError):
        fbg.quantize_rows(torch.zeros(4, 128, dtype=torch.bfloat16))      # not on a GPU


def _bcall(w=0x100000, N=300, K=256, B=0x200000, b_s=0x300000):
    return fbg.load().fp8_block_gemm_quantize_blocks(w, N, K, B, b_s, None)


def test_quantize_blocks_host_validation_statuses():
    assert _bcall(w=None) == fbg.INVALID_VALUE
    assert _bcall(B=None) == fbg.INVALID_VALUE
    assert _bcall(b_s=None) == fbg.INVALID_VALUE
    assert _bcall(N=-1) == fbg.INVALID_VALUE
    assert _bcall(K=130) == fbg.UNSUPPORTED
    assert _bcall(w=0x100004) == fbg.UNSUPPORTED
    assert _bcall(B=0x200002) == fbg.UNSUPPORTED
    assert _bcall(b_s=0x300001) == fbg.UNSUPPORTED
    assert _bcall(B=0x100000 + 4096) == fbg.INVALID_VALUE     # B overlaps w (300*256*2 bytes)
    assert _bcall(N=0, w=None, B=None, b_s=None) == fbg.SUCCESS
    with pytest.raises(ValueError):
        fbg.quantize_blocks(torch.zeros(4, 128, dtype=torch.bfloat16))


def _gcall(A=0x100000, a_s=0x200000, B=0x300000, b_s=0x400000, C=0x50000000, off=0x600000, E=4, M=16, N=256,
           K=256, out=0):
    return fbg.load().fp8_block_gemm_grouped(A, a_s, B, b_s, C, off, E, M, N, K, out, None)


def test_grouped_host_validation_statuses():
    # As above: every case fails validation (or is empty) before any HIP call.
    assert _gcall(A=None) == fbg.INVALID_VALUE
    assert _gcall(a_s=None) == fbg.INVALID_VALUE
    assert _gcall(B=None) == fbg.INVALID_VALUE
    assert _gcall(b_s=None) == fbg.INVALID_VALUE
    assert _gcall(C=None) == fbg.INVALID_VALUE
    assert _gcall(off=None) == fbg.INVALID_VALUE
    assert _gcall(E=-1) == fbg.INVALID_VALUE
    assert _gcall(M=-1) == fbg.INVALID_VALUE
    assert _gcall(out=5) == fbg.INVALID_VALUE
    assert _gcall(K=200) == fbg.UNSUPPORTED
    assert _gcall(K=(1 << 24) + 128) == fbg.UNSUPPORTED
    assert _gcall(K=1 << 24) == fbg.UNSUPPORTED
    assert _gcall(A=0x100008) == fbg.UNSUPPORTED            # A not 16-byte aligned
    assert _gcall(B=0x300004) == fbg.UNSUPPORTED
    assert _gcall(b_s=0x400002) == fbg.UNSUPPORTED
    assert _gcall(off=0x600002) == fbg.UNSUPPORTED          # offsets not 4-byte aligned
    assert _gcall(C=0x50000001) == fbg.UNSUPPORTED
    assert _gcall(C=0x300000 + 4096) == fbg.INVALID_VALUE   # C overlaps B (4*256*256 bytes)
    assert _gcall(C=0x600000 - 64) == fbg.INVALID_VALUE     # C overlaps the offsets
    assert _gcall(M=0, A=None, a_s=None, C=None) == fbg.SUCCESS   # empty: nothing launched
    assert _gcall(N=0, B=None, b_s=None, C=None) == fbg.SUCCESS
    assert _gcall(E=1 << 30, N=1 << 30, K=1 << 30) == fbg.UNSUPPORTED   # E*N*K overflows int64
    assert _gcall(M=1 << 31) == fbg.UNSUPPORTED                          # above INT32_MAX
    assert _call(M=(1 << 31) - 1, K=1 << 20) == fbg.UNSUPPORTED          # a_s of 64 GiB: past 32-bit offsets


def test_grouped_wrapper_checks():
    A = torch.zeros((5, 256), dtype=torch.float8_e4m3fn)
    B = torch.zeros((2, 130, 256), dtype=torch.float8_e4m3fn)
    a_s, b_s = torch.zeros((5, 2)), torch.zeros((2, 2, 2))
    with pytest.raises(ValueError):       # offsets need E + 1 entries
        fbg.grouped_gemm(A, a_s, B, b_s, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(TypeError):
        fbg.grouped_gemm(A, a_s, B, b_s, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError):       # B must be [E, N, K]
        fbg.grouped_gemm(A, a_s, B[0], b_s, torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError):
        fbg.grouped_gemm(A, a_s, B, torch.zeros((2, 1, 2)), torch.zeros(3, dtype=torch.int32))


def test_grouped_plan():
    for E, M, N in [(256, 128, 512), (256, 512, 512), (256, 8192, 512), (7, 100, 300), (1, 5, 130)]:  # skinny
        p = fbg.grouped_plan(E, M, N, 1024)
        assert p["variant_name"] == "grouped" and p["split_k"] == 1 and p["workspace_bytes"] == 0
        assert p["grid"] == E * -(-N // p["tile_n"])
        assert 128 % p["tile_n"] == 0 and p["tile_m"] % 16 == 0
    # more tokens per expert -> taller tiles; prefill-sized experts on the
    # generic kernel, whose grid bounds the experts' row tiles by
    # ceil(M / BM) + E
    assert fbg.grouped_plan(256, 8192, 512, 4096)["tile_m"] > fbg.grouped_plan(256, 512, 512, 4096)["tile_m"]
    p = fbg.grouped_plan(256, 16384, 512, 4096)   # ~64 rows per expert: 128 x 256 tiles
    assert (p["tile_m"], p["tile_n"], p["waves"]) == (128, 256, 8)
    assert p["grid"] == (-(-16384 // 128) + 256) * 2
    p = fbg.grouped_plan(256, 32768, 512, 4096)
    assert p["tile_m"] == 256 and p["waves"] == 8
    assert p["grid"] == (-(-32768 // 256) + 256) * -(-512 // p["tile_n"])
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.grouped_plan(-1, 5, 130, 256)
    assert e.value.status == fbg.INVALID_VALUE
    with pytest.raises(fbg.FP8BGError) as e:
        fbg.grouped_plan(2, 5, 130, 200)
    assert e.value.status == fbg.UNSUPPORTED


def test_header_is_plain_c_and_matches_the_library(tmp_path):
    """include/fp8bg.h compiles as C99 and C++ on its own, and a C program
    that calls every declared function's address links against the library
    (signatures as declared, C linkage)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "use.c"
    src.write_text('#include "fp8bg.h"\n#include <stdio.h>\nint main(void) {\n'
                   + "".join(f'  printf("%p\\n", (void *)&{n});\n' for n in names)
                   + "  fbg_plan p;\n  return fp8_block_gemm_plan(64, 512, 4096, FBG_OUT_BF16, 256, FBG_VARIANT_AUTO, 0, &p)"
                     " == FBG_SUCCESS && p.split_k >= 1 ? 0 : 1;\n}\n")
    lib = os.path.join(ROOT, "block_scaled_fp8_gemm_amd")
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", lib, "-lfp8bg", "-Wl,-rpath," + lib, "-o", str(exe)], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++",
                    "-I", os.path.join(ROOT, "include"), str(src)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert len(r.stdout.split()) == len(names)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more exits with status 2 and
    a JSON line that says why, before touching any device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_probe_library_rejects_bad_arguments_before_any_launch():
    """The load-path probe (a measuring tool beside the library) checks its
    region against the caller's buffer on the host; a rejected call returns 1
    and makes no HIP call."""
    lib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_fp8_gemm_amd", "libfp8bg_probe.so"))
    f = lib.fbg_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is rejected first
    assert f(None, 1 << 20, 0, 1 << 20, 256, 4, 1, 64, fake, None) == 1           # no source
    assert f(fake, 1 << 20, 0, 3 << 10, 256, 4, 1, 64, fake, None) == 1           # region not a power of two
    assert f(fake, 1 << 20, 0, 512, 256, 4, 1, 64, fake, None) == 1               # region below 1 KB
    assert f(fake, 256 << 20, 1 << 20, 1 << 20, 257, 4, 1, 64, fake, None) == 1   # last region past the buffer
    assert f(fake, 256 << 20, 1 << 20, 1 << 20, 256, 4, 1, 0, fake, None) == 1    # no loads
    assert f(fake, 256 << 20, 1 << 20, 1 << 20, 256, 5, 1, 64, fake, None) == 1   # 4 or 8 waves only
