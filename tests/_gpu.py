"""Helpers for the GPU parity tests: move seeded numpy inputs to cuda:0, run
the HIP path through the C ABI, and compare with the oracle."""
import contextlib
import os

import numpy as np
import torch

import oracle

TORCH_OUT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
BITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32}


def to_dev(d):
    dev = torch.device("cuda:0")
    return {
        "A": torch.from_numpy(np.ascontiguousarray(d["A"])).to(dev).view(torch.float8_e4m3fn),
        "a_s": torch.from_numpy(np.ascontiguousarray(d["a_s"])).to(dev),
        "B": torch.from_numpy(np.ascontiguousarray(d["B"])).to(dev).view(torch.float8_e4m3fn),
        "b_s": torch.from_numpy(np.ascontiguousarray(d["b_s"])).to(dev),
    }


@contextlib.contextmanager
def forced_config(cfg):
    old = os.environ.get("FBG_FORCE_CONFIG")
    if cfg is None:
        os.environ.pop("FBG_FORCE_CONFIG", None)
    else:
        os.environ["FBG_FORCE_CONFIG"] = str(cfg)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("FBG_FORCE_CONFIG", None)
        else:
            os.environ["FBG_FORCE_CONFIG"] = old


def run(fbg, dd, out="bf16", variant="auto", split_k=0, cfg=None, workspace=None, C=None, stream=None):
    with forced_config(cfg):
        C = fbg.gemm(dd["A"], dd["a_s"], dd["B"], dd["b_s"], out_dtype=TORCH_OUT[out], variant=variant,
                     split_k=split_k, workspace=workspace, out=C, stream=stream)
    torch.cuda.synchronize()
    return C


def bits(C, out):
    return C.contiguous().cpu().view(torch.int16 if out != "fp32" else torch.int32).numpy().view(BITS[out])


def as_f64(C):
    return C.float().cpu().double().numpy()


def assert_within_tolerance(C, ref, out, what=""):
    """|C - C_ref| <= 2 ulp_dtype(|C_ref|) + 1e-3 rms(C_ref), elementwise."""
    got = as_f64(C)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol = oracle.tolerance(ref, out)
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {idx.tolist()}, "
                             f"max err {err.max():.4g}, got {got[tuple(idx[0])]:.6g} want {ref[tuple(idx[0])]:.6g}")
    return float(err.max())


def assert_bitwise(C, ref64, out, what=""):
    want = oracle.round_bits(ref64, out)
    got = bits(C, out)
    diff = got != want
    if diff.any():
        idx = np.argwhere(diff)[:5]
        raise AssertionError(f"{what}: {int(diff.sum())} of {diff.size} differ bitwise; first {idx.tolist()}, "
                             f"got {got[tuple(idx[0])]:#x} want {want[tuple(idx[0])]:#x}")
