"""CPU oracle for the W8A8 block-scaled FP8 matmul.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The GPU product path
never imports this package.

The arithmetic lives in ``fp8bg_oracle.c`` (plain C, fp64); this module only
marshals numpy arrays into it.  What is computed (FlagGems-vllm PR #693,
"feat: optimize w8a8 block fp8 matmul for Hopper", sections "Description" and
"Numerical safety"):

    C[m,n] = sum_g a_s[m,g] * b_s[n//128, g] * sum_{k in group g} A[m,k] * B[n,k]

Every function here is pinned by tests in ``tests/test_oracle_*.py``
(brute force with exact rationals, integer-valued inputs checked against
int64 arithmetic, numpy fp64 BLAS cross-checks, special cases and
invariants); no function is left with its parity unpinned.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")

BF16, FP16, FP32 = 0, 1, 2
DTYPE_CODES = {"bf16": BF16, "fp16": FP16, "fp32": FP32}
GROUP = 128

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from oracle import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.fp8bg_oracle_e4m3_value.restype = ctypes.c_double
    lib.fp8bg_oracle_e4m3_value.argtypes = [ctypes.c_uint]
    lib.fp8bg_oracle_gemm.restype = None
    lib.fp8bg_oracle_gemm.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p]
    lib.fp8bg_oracle_round.restype = ctypes.c_int
    lib.fp8bg_oracle_round.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.fp8bg_oracle_e4m3_encode.restype = ctypes.c_uint
    lib.fp8bg_oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.fp8bg_oracle_quantize_rows.restype = None
    lib.fp8bg_oracle_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_void_p]
    lib.fp8bg_oracle_quantize_blocks.restype = None
    lib.fp8bg_oracle_quantize_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.fp8bg_oracle_threads.restype = ctypes.c_int
    lib.fp8bg_oracle_threads.argtypes = []
    lib.fp8bg_oracle_set_threads.restype = None
    lib.fp8bg_oracle_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _dtype_code(out_dtype):
    if isinstance(out_dtype, int):
        return out_dtype
    return DTYPE_CODES[out_dtype]


def e4m3_value(code: int) -> float:
    """Exact value of one OCP E4M3 code (NaN for 0x7F / 0xFF)."""
    return _load().fp8bg_oracle_e4m3_value(int(code) & 0xFF)


def e4m3_table() -> np.ndarray:
    """fp64 values of all 256 E4M3 codes, indexed by code."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def block_gemm(A, a_s, B, b_s) -> np.ndarray:
    """fp64 C[M,N] of the block-scaled GEMM.

    A: uint8 [M,K] E4M3 codes; B: uint8 [N,K]; a_s: float32 [M, ceil(K/128)];
    b_s: float32 [ceil(N/128), ceil(K/128)].  All C-contiguous.
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    G = (K + GROUP - 1) // GROUP
    NB = (N + GROUP - 1) // GROUP
    if a_s.shape != (M, G) or b_s.shape != (NB, G):
        raise ValueError(f"scale shapes {a_s.shape}, {b_s.shape}; expected {(M, G)}, {(NB, G)}")
    C = np.empty((M, N), dtype=np.float64)
    if M and N:
        _load().fp8bg_oracle_gemm(A.ctypes.data, a_s.ctypes.data, B.ctypes.data,
                                  b_s.ctypes.data, M, N, K, C.ctypes.data)
    return C


def grouped_gemm(A, a_s, B, b_s, offsets) -> np.ndarray:
    """fp64 C[M,N] of the grouped (mixture-of-experts) block-scaled GEMM: the
    rows offsets[e] .. offsets[e+1]-1 of A are the tokens routed to expert e
    and are multiplied by that expert's weight B[e] with its block scales
    b_s[e] -- the block-scaled GEMM of this module, once per expert (the
    MoE-style traffic the first page's "Description" names; the expert
    weights and per-expert token groups of the MoE kernel page).

    A: uint8 [M,K]; a_s: float32 [M,G]; B: uint8 [E,N,K]; b_s: float32
    [E, ceil(N/128), G]; offsets: E+1 non-decreasing integers from 0 to M.
    """
    B = np.ascontiguousarray(B, dtype=np.uint8)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    offsets = np.asarray(offsets, dtype=np.int64)
    E, N, K = B.shape
    M = A.shape[0]
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != M or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be E+1 non-decreasing integers from 0 to M")
    C = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            C[r0:r1] = block_gemm(A[r0:r1], a_s[r0:r1], B[e], b_s[e])
    return C


def round_bits(x, out_dtype) -> np.ndarray:
    """One-step RNE of fp64 values to out_dtype; returns the bit patterns
    (uint16 for bf16/fp16, uint32 for fp32) with x's shape."""
    code = _dtype_code(out_dtype)
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32 if code == FP32 else np.uint16)
    rc = _load().fp8bg_oracle_round(x.ctypes.data, x.size, code, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"unknown dtype code {code}")
    return out


def bits_to_f64(bits, out_dtype) -> np.ndarray:
    """Decodes bf16/fp16/fp32 bit patterns to fp64 (plain IEEE bit reinterpretation)."""
    code = _dtype_code(out_dtype)
    bits = np.asarray(bits)
    if code == FP32:
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if code == FP16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def threads() -> int:
    """Threads the oracle's OpenMP loop uses."""
    return int(_load().fp8bg_oracle_threads())


def set_threads(n: int) -> None:
    """Sets the oracle's OpenMP thread count (for timing only; results do not
    depend on it: every output element is computed by one thread)."""
    _load().fp8bg_oracle_set_threads(int(n))


# (precision p incl. hidden bit, minimum normal exponent) per output dtype
_FORMAT = {BF16: (8, -126), FP16: (11, -14), FP32: (24, -126)}


def ulp(x, out_dtype) -> np.ndarray:
    """Spacing of out_dtype at |x|: 2^(max(floor(log2|x|), e_min) - p + 1)."""
    p, emin = _FORMAT[_dtype_code(out_dtype)]
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)                        # a = f * 2^e, f in [0.5, 1): floor(log2 a) = e - 1
    e = np.maximum(np.where(a > 0, e.astype(np.int64) - 1, emin), emin)
    return np.ldexp(1.0, e - p + 1)


def tolerance(C_ref, out_dtype) -> np.ndarray:
    """Elementwise bound |C - C_ref| <= 2 ulp_dtype(|C_ref|) + 1e-3 * rms(C_ref)."""
    C_ref = np.asarray(C_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(np.square(C_ref)))) if C_ref.size else 0.0
    return 2.0 * ulp(C_ref, out_dtype) + 1e-3 * rms


def e4m3_encode(x: float) -> int:
    """OCP E4M3 code of a finite value, round to nearest even, saturating at
    +-448 (fp8bg_oracle.c, fp8bg_oracle_e4m3_encode)."""
    return int(_load().fp8bg_oracle_e4m3_encode(float(x)))


def quantize_rows(x_bf16_bits):
    """Per-token 1 x 128 activation quantisation (FlagGems-vllm PR #693,
    section "Description": FP8 E4M3 activations with per-token scales).

    x_bf16_bits: uint16 [M,K] bf16 bit patterns.  Returns (A, a_s): uint8
    [M,K] E4M3 codes and float32 [M, ceil(K/128)] scales, with
    a_s = max(amax, 1e-12)/448 per group and A = E4M3_RNE(clamp(x/a_s, +-448)),
    both divisions in fp32.
    """
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    G = (K + GROUP - 1) // GROUP
    q = np.empty((M, K), dtype=np.uint8)
    a_s = np.empty((M, G), dtype=np.float32)
    if M and K:
        _load().fp8bg_oracle_quantize_rows(x.ctypes.data, M, K, q.ctypes.data, a_s.ctypes.data)
    return q, a_s


def quantize_blocks(w_bf16_bits):
    """128 x 128 block quantisation of bf16 weights (FlagGems-vllm PR #693,
    section "Description": FP8 E4M3 weights with [block_n, block_k] = [128, 128]
    de-quant scales).

    w_bf16_bits: uint16 [N,K] bf16 bit patterns.  Returns (B, b_s): uint8 [N,K]
    E4M3 codes and float32 [ceil(N/128), ceil(K/128)] scales, with
    b_s = max(amax, 1e-12)/448 per block and B = E4M3_RNE(clamp(w/b_s, +-448)),
    both divisions in fp32.
    """
    w = np.ascontiguousarray(w_bf16_bits, dtype=np.uint16)
    N, K = w.shape
    NB, G = (N + GROUP - 1) // GROUP, (K + GROUP - 1) // GROUP
    q = np.empty((N, K), dtype=np.uint8)
    b_s = np.empty((NB, G), dtype=np.float32)
    if N and K:
        _load().fp8bg_oracle_quantize_blocks(w.ctypes.data, N, K, q.ctypes.data, b_s.ctypes.data)
    return q, b_s
