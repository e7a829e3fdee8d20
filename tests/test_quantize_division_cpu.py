"""The activation quantiser's GPU kernel replaces the per-element fp32
division x / a_s by a per-group reciprocal and one correction step.  This
CPU test runs tests/quantize_division_check.c, which compares the E4M3 code
of both quotients for every possible (bf16 x, bf16 group maximum) pair --
about 1.07e9 pairs -- and fails on any difference.  (The per-token scale
recipe: FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for
Hopper", section "Description".)
"""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_reciprocal_and_correction_give_the_division_codes():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "check")
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-std=c11",
                        os.path.join(ROOT, "tests", "quantize_division_check.c"),
                        os.path.join(ROOT, "oracle", "fp8bg_oracle.c"), "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    pairs = int(r.stdout.split()[1])
    assert pairs > 1_000_000_000, r.stdout
