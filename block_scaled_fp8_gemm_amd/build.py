"""Builds the HIP library libfp8bg.so in-tree for gfx950 with hipcc, and
beside it libfp8bg_probe.so, the load-path probe that the benchmark's
--probe-load mode runs (a measuring tool, not part of the GEMM library).

Every HIP source is compiled for gfx950 only.  Flags:
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-FP32 VALU ops
  -ffp-contract=off                                   only the FMAs written in the source
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8bg.so")
SOURCES = ["fp8bg_api.hip", "fp8bg_kernels.hip", "fp8bg_quant.hip", "fp8bg_plan.cpp"]
PROBE_LIB = os.path.join(PKG, "libfp8bg_probe.so")
PROBE_SOURCES = ["fp8bg_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wall", "-Wno-unused-function",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False, jobs: int = 3) -> str:
    lib = _build_lib(SOURCES, LIB, verbose, jobs)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose, jobs)
    return lib


def _build_lib(sources, out, verbose: bool, jobs: int) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
        while len([p for p, _ in procs if p.poll() is None]) >= jobs:
            procs[0][0].wait()
    for p, src in procs:
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {src}")
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    # A kernel whose host launch stub was not emitted links fine into a
    # shared library and only fails at load time: refuse it here.
    nm = subprocess.run(["nm", "-D", "--undefined-only", out + ".tmp"], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub" in l]
    if missing:
        raise RuntimeError(f"kernel launch stubs missing from the library: {missing[:3]}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
