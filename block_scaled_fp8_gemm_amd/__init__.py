"""Python binding of libfp8bg.so, the gfx950 block-scaled FP8 GEMM library.

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels; torch supplies device memory and the current stream.  The C ABI is
declared in include/fp8bg.h.

    C[m,n] = sum_g a_s[m,g] * b_s[n//128,g] * sum_{k in g} A[m,k] * B[n,k]

(FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul for Hopper",
section "Description".)  If the library is not built, load() raises: there is
no fallback of any kind.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8bg.so")

SUCCESS, INVALID_VALUE, UNSUPPORTED, OUT_OF_MEMORY, HIP_ERROR, SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5
VARIANTS = {"auto": 0, "generic": 1, "short_k256": 2, "swap_ab": 3, "swap_ab_splitk": 4}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
VARIANT_NAMES[5] = "grouped"          # reported by grouped_plan only
OUT_CODES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
OUT_DTYPES = {v: k for k, v in OUT_CODES.items()}
FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


class FP8BGError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("waves", ctypes.c_int32), ("config", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


_lib = None
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


def load():
    """Loads libfp8bg.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fp8_block_gemm.restype = _int
    lib.fp8_block_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]
    lib.fp8_block_gemm_ex.restype = _int
    lib.fp8_block_gemm_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp,
                                      _int, _int, _vp, _sz]
    lib.fp8_block_gemm_noalloc.restype = _int
    lib.fp8_block_gemm_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _int, _int]
    lib.fp8_block_gemm_workspace_size.restype = _sz
    lib.fp8_block_gemm_workspace_size.argtypes = [_i64, _i64, _i64, _int, _int]
    lib.fp8_block_gemm_plan.restype = _int
    lib.fp8_block_gemm_plan.argtypes = [_i64, _i64, _i64, _int, _int, _int, _int, ctypes.POINTER(Plan)]
    lib.fp8_block_gemm_status_string.restype = ctypes.c_char_p
    lib.fp8_block_gemm_status_string.argtypes = [_int]
    lib.fp8_block_gemm_quantize_rows.restype = _int
    lib.fp8_block_gemm_quantize_rows.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    lib.fp8_block_gemm_quantize_blocks.restype = _int
    lib.fp8_block_gemm_quantize_blocks.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    lib.fp8_block_gemm_grouped.restype = _int
    lib.fp8_block_gemm_grouped.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]
    lib.fp8_block_gemm_grouped_plan.restype = _int
    lib.fp8_block_gemm_grouped_plan.argtypes = [_i64, _i64, _i64, _i64, _vp]
    lib.fp8_block_gemm_version.restype = _int
    lib.fp8_block_gemm_version.argtypes = []
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fp8_block_gemm_status_string(int(status)).decode()


def _variant_code(variant) -> int:
    return VARIANTS[variant] if isinstance(variant, str) else int(variant)


def _out_code(out_dtype) -> int:
    if isinstance(out_dtype, int):
        return out_dtype
    return OUT_CODES[out_dtype]


def plan(M: int, N: int, K: int, out_dtype=torch.bfloat16, cu_count: int = 256,
         variant="auto", split_k: int = 0) -> dict:
    """The dispatcher's decision (pure host call; works without a GPU)."""
    p = Plan()
    st = load().fp8_block_gemm_plan(M, N, K, _out_code(out_dtype), cu_count, _variant_code(variant),
                                    split_k, ctypes.byref(p))
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_plan")
    d = {f: getattr(p, f) for f, _ in Plan._fields_}
    d["variant_name"] = VARIANT_NAMES.get(p.variant, "none")
    return d


def grouped_plan(E: int, M: int, N: int, K: int) -> dict:
    """The grouped GEMM's tile choice for E experts holding M rows (pure host call)."""
    p = Plan()
    st = load().fp8_block_gemm_grouped_plan(E, M, N, K, ctypes.byref(p))
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_grouped_plan")
    d = {f: getattr(p, f) for f, _ in Plan._fields_}
    d["variant_name"] = VARIANT_NAMES.get(p.variant, "none")
    return d


def workspace_size(M: int, N: int, K: int, variant="auto", split_k: int = 0) -> int:
    n = load().fp8_block_gemm_workspace_size(M, N, K, _variant_code(variant), split_k)
    if n == ctypes.c_size_t(-1).value:
        raise FP8BGError(INVALID_VALUE, "fp8_block_gemm_workspace_size")
    return int(n)


def _check(t, name, dtypes, shape, device):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def gemm(A: torch.Tensor, a_s: torch.Tensor, B: torch.Tensor, b_s: torch.Tensor,
         out_dtype=torch.bfloat16, out: torch.Tensor = None, variant="auto", split_k: int = 0,
         workspace: torch.Tensor = None, stream: torch.cuda.Stream = None) -> torch.Tensor:
    """C = block-scaled A @ B^T on the current stream (or `stream`).

    A [M,K] and B [N,K]: float8_e4m3fn (or uint8 holding E4M3 codes);
    a_s [M, K/128], b_s [ceil(N/128), K/128]: float32; all contiguous on one
    GPU.  variant/split_k force a kernel (see include/fp8bg.h).  workspace:
    None (default) -- when the plan splits K, a zeroed byte tensor from
    torch's caching allocator on the call's stream (cheap, and captured into
    a HIP graph's memory pool like any tensor); "library" -- the C library's
    own stream-ordered allocation (fp8_block_gemm), whose allocation and free
    become graph nodes under capture; or a caller-owned byte tensor whose
    counter area is zero.
    """
    lib = load()
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    G, NB = (K + 127) // 128, (N + 127) // 128
    dev = A.device
    _check(A, "A", FP8_DTYPES, (M, K), dev)
    _check(B, "B", FP8_DTYPES, (N, K), dev)
    _check(a_s, "a_s", (torch.float32,), (M, G), dev)
    _check(b_s, "b_s", (torch.float32,), (NB, G), dev)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _check(out, "out", (out_dtype,), (M, N), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    v, code = _variant_code(variant), _out_code(out_dtype)
    if isinstance(workspace, str):
        if workspace != "library":
            raise ValueError('workspace must be None, "library" or a byte tensor')
        workspace = None
    elif workspace is None:
        need = lib.fp8_block_gemm_workspace_size(M, N, K, v, split_k)
        if 0 < need < ctypes.c_size_t(-1).value:   # an invalid request is reported by the call itself
            with torch.cuda.stream(s):
                workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    if v == 0 and split_k == 0 and workspace is None:
        st = lib.fp8_block_gemm(A.data_ptr(), a_s.data_ptr(), B.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                                M, N, K, code, s.cuda_stream)
    else:
        wp, wn = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) \
            if workspace is not None else (None, 0)
        st = lib.fp8_block_gemm_ex(A.data_ptr(), a_s.data_ptr(), B.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                                   M, N, K, code, s.cuda_stream, v, split_k, wp, wn)
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm")
    return out


def gemm_noalloc(A: torch.Tensor, a_s: torch.Tensor, B: torch.Tensor, b_s: torch.Tensor,
                 out: torch.Tensor, variant="auto", split_k: int = 0,
                 stream: torch.cuda.Stream = None) -> torch.Tensor:
    """fp8_block_gemm_noalloc: the GEMM with any split-K partials in the
    library's static per-GPU scratch, for callers that cannot allocate.  `out`
    is required (this call allocates nothing, not even its output).  Calls
    that overlap in time on one GPU share the scratch and must not be made;
    see include/fp8bg.h."""
    lib = load()
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    G, NB = (K + 127) // 128, (N + 127) // 128
    dev = A.device
    _check(A, "A", FP8_DTYPES, (M, K), dev)
    _check(B, "B", FP8_DTYPES, (N, K), dev)
    _check(a_s, "a_s", (torch.float32,), (M, G), dev)
    _check(b_s, "b_s", (torch.float32,), (NB, G), dev)
    if out is None or out.dtype not in OUT_CODES:
        raise ValueError("out must be a bf16 / fp16 / fp32 tensor")
    _check(out, "out", (out.dtype,), (M, N), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib.fp8_block_gemm_noalloc(A.data_ptr(), a_s.data_ptr(), B.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                                    M, N, K, OUT_CODES[out.dtype], s.cuda_stream, _variant_code(variant), split_k)
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_noalloc")
    return out


def quantize_rows(x: torch.Tensor, A: torch.Tensor = None, a_s: torch.Tensor = None,
                  stream: torch.cuda.Stream = None):
    """Per-token 1x128 quantisation of bf16 activations x [M,K] into E4M3 codes
    A [M,K] (float8_e4m3fn) and fp32 scales a_s [M, K/128], on the current
    stream (or `stream`): a_s = max(amax, 1e-12)/448 per 128-wide group,
    A = E4M3_RNE(clamp(x / a_s, +-448)).  See fp8_block_gemm_quantize_rows in
    include/fp8bg.h."""
    lib = load()
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous 2-D bfloat16 CUDA tensor")
    M, K = x.shape
    G = (K + 127) // 128
    if A is None:
        A = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    else:
        _check(A, "A", FP8_DTYPES, (M, K), x.device)
    if a_s is None:
        a_s = torch.empty((M, G), dtype=torch.float32, device=x.device)
    else:
        _check(a_s, "a_s", (torch.float32,), (M, G), x.device)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    st = lib.fp8_block_gemm_quantize_rows(x.data_ptr(), M, K, A.data_ptr(), a_s.data_ptr(), s.cuda_stream)
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_quantize_rows")
    return A, a_s


def quantize_blocks(w: torch.Tensor, B: torch.Tensor = None, b_s: torch.Tensor = None,
                    stream: torch.cuda.Stream = None):
    """128x128 block quantisation of bf16 weights w [N,K] into E4M3 codes
    B [N,K] (float8_e4m3fn) and fp32 scales b_s [ceil(N/128), K/128]:
    b_s = max(amax, 1e-12)/448 per block, B = E4M3_RNE(clamp(w / b_s, +-448)).
    See fp8_block_gemm_quantize_blocks in include/fp8bg.h."""
    lib = load()
    if w.dim() != 2 or w.dtype != torch.bfloat16 or not w.is_contiguous() or not w.is_cuda:
        raise ValueError("w must be a contiguous 2-D bfloat16 CUDA tensor")
    N, K = w.shape
    NB, G = (N + 127) // 128, (K + 127) // 128
    if B is None:
        B = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
    else:
        _check(B, "B", FP8_DTYPES, (N, K), w.device)
    if b_s is None:
        b_s = torch.empty((NB, G), dtype=torch.float32, device=w.device)
    else:
        _check(b_s, "b_s", (torch.float32,), (NB, G), w.device)
    s = stream if stream is not None else torch.cuda.current_stream(w.device)
    st = lib.fp8_block_gemm_quantize_blocks(w.data_ptr(), N, K, B.data_ptr(), b_s.data_ptr(), s.cuda_stream)
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_quantize_blocks")
    return B, b_s


def grouped_gemm(A: torch.Tensor, a_s: torch.Tensor, B: torch.Tensor, b_s: torch.Tensor, offsets: torch.Tensor,
                 out_dtype=torch.bfloat16, out: torch.Tensor = None, stream: torch.cuda.Stream = None) -> torch.Tensor:
    """Grouped (mixture-of-experts) block-scaled GEMM: rows offsets[e] ..
    offsets[e+1]-1 of A use expert e's weight B[e] [N,K] and scales b_s[e].

    A [M,K] E4M3, a_s [M,K/128] fp32, B [E,N,K] E4M3, b_s [E,ceil(N/128),K/128]
    fp32, offsets int32 [E+1] on the same GPU.  See fp8_block_gemm_grouped in
    include/fp8bg.h."""
    lib = load()
    if A.dim() != 2 or B.dim() != 3:
        raise ValueError("A must be 2-D and B 3-D [E, N, K]")
    M, K = A.shape
    E, N = B.shape[0], B.shape[1]
    G, NB = (K + 127) // 128, (N + 127) // 128
    dev = A.device
    _check(A, "A", FP8_DTYPES, (M, K), dev)
    _check(B, "B", FP8_DTYPES, (E, N, K), dev)
    _check(a_s, "a_s", (torch.float32,), (M, G), dev)
    _check(b_s, "b_s", (torch.float32,), (E, NB, G), dev)
    _check(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _check(out, "out", (out_dtype,), (M, N), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    st = lib.fp8_block_gemm_grouped(A.data_ptr(), a_s.data_ptr(), B.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                                    offsets.data_ptr(), E, M, N, K, _out_code(out_dtype), s.cuda_stream)
    if st != SUCCESS:
        raise FP8BGError(st, "fp8_block_gemm_grouped")
    return out
