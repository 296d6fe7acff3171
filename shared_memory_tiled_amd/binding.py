"""Python binding of libgemm_f32.so (argument marshalling only).

The functions mirror the C entry points of ``include/gemm_f32.h`` one to one;
every step of the product runs in the library's HIP kernels.  torch provides
device memory and streams: matrix arguments may be torch CUDA tensors (their
``data_ptr()``, which includes any storage offset) or raw device addresses.

torch is imported before the library is loaded so that both use torch's HIP
runtime.  There is no fallback: if the library is missing and cannot be
built, or a call returns a nonzero status, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must precede loading the HIP library)

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libgemm_f32.so")

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib = None
_lock = threading.Lock()

OK = 0
VARIANTS = {"naive": 0, "tiled": 1, "regblock": 2, "mfma": 3}
OPS = {"N": 0, "T": 1, 0: 0, 1: 1}
DIAGNOSTIC_BASE = 16


class GemmError(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"gemm_f32 status {status}: {message}")
        self.status = status


def load_library():
    """Loads libgemm_f32.so, building it only if no built library exists."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(library_path):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(library_path)
        sig = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
        lib.gemm_f32.argtypes = sig
        lib.gemm_f32.restype = ctypes.c_int
        lib.gemm_f32_variant.argtypes = [ctypes.c_int] + sig
        lib.gemm_f32_variant.restype = ctypes.c_int
        lib.gemm_f32_op.argtypes = [ctypes.c_int, ctypes.c_int] + sig
        lib.gemm_f32_op.restype = ctypes.c_int
        lib.gemm_f32_num_variants.argtypes = []
        lib.gemm_f32_num_variants.restype = ctypes.c_int
        lib.gemm_f32_num_diagnostic_variants.argtypes = []
        lib.gemm_f32_num_diagnostic_variants.restype = ctypes.c_int
        lib.gemm_f32_variant_name.argtypes = [ctypes.c_int]
        lib.gemm_f32_variant_name.restype = ctypes.c_char_p
        lib.gemm_f32_status_string.argtypes = [ctypes.c_int]
        lib.gemm_f32_status_string.restype = ctypes.c_char_p
        lib.gemm_f32_default_variant.argtypes = [_i64, _i64, _i64]
        lib.gemm_f32_default_variant.restype = ctypes.c_int
        tsig = [_i64, _i64, _vp, _i64, _vp, _i64, _vp]
        lib.transpose_f32.argtypes = tsig
        lib.transpose_f32.restype = ctypes.c_int
        lib.transpose_f32_variant.argtypes = [ctypes.c_int] + tsig
        lib.transpose_f32_variant.restype = ctypes.c_int
        lib.transpose_f32_num_variants.argtypes = []
        lib.transpose_f32_num_variants.restype = ctypes.c_int
        lib.transpose_f32_variant_name.argtypes = [ctypes.c_int]
        lib.transpose_f32_variant_name.restype = ctypes.c_char_p
        lib.transpose_f32_default_variant.argtypes = [_i64, _i64, _i64, _i64]
        lib.transpose_f32_default_variant.restype = ctypes.c_int
        lib.reduce_sum_f32_workspace_size.argtypes = [ctypes.c_int, _i64]
        lib.reduce_sum_f32_workspace_size.restype = _i64
        rsig = [_i64, _vp, _vp, _vp, _i64, _vp]
        lib.reduce_sum_f32.argtypes = rsig
        lib.reduce_sum_f32.restype = ctypes.c_int
        lib.reduce_sum_f32_variant.argtypes = [ctypes.c_int] + rsig
        lib.reduce_sum_f32_variant.restype = ctypes.c_int
        lib.gemm_f32_valu_probe.argtypes = [ctypes.c_int, _i64, ctypes.c_int, _vp, _vp, _vp]
        lib.gemm_f32_valu_probe.restype = ctypes.c_int
        lib.gemm_f32_lds_probe.argtypes = [ctypes.c_int, _vp, ctypes.c_int, _vp, _vp]
        lib.gemm_f32_lds_probe.restype = ctypes.c_int
        lib.gemm_f32_copy_probe.argtypes = [ctypes.c_int, _i64, ctypes.c_int, _vp, _vp, _vp, _vp]
        lib.gemm_f32_copy_probe.restype = ctypes.c_int
        lib.gemm_f32_ksplit_timeline.argtypes = sig[:-1] + [_vp, _i64, _vp]
        lib.gemm_f32_ksplit_timeline.restype = ctypes.c_int
        lib.reduce_sum_f32_variant_noalloc.argtypes = [ctypes.c_int, _i64, _vp, _vp, _vp]
        lib.reduce_sum_f32_variant_noalloc.restype = ctypes.c_int
        lib.reduce_sum_f32_num_variants.argtypes = []
        lib.reduce_sum_f32_num_variants.restype = ctypes.c_int
        lib.reduce_sum_f32_variant_name.argtypes = [ctypes.c_int]
        lib.reduce_sum_f32_variant_name.restype = ctypes.c_char_p
        msig = [ctypes.c_int] + sig
        lib.gemm_mixed.argtypes = msig
        lib.gemm_mixed.restype = ctypes.c_int
        lib.gemm_mixed_variant.argtypes = [ctypes.c_int] + msig
        lib.gemm_mixed_variant.restype = ctypes.c_int
        lib.gemm_mixed_op.argtypes = [ctypes.c_int, ctypes.c_int] + msig
        lib.gemm_mixed_op.restype = ctypes.c_int
        lib.gemm_mixed_num_variants.argtypes = []
        lib.gemm_mixed_num_variants.restype = ctypes.c_int
        lib.gemm_mixed_default_variant.argtypes = [_i64, _i64, _i64]
        lib.gemm_mixed_default_variant.restype = ctypes.c_int
        lib.gemm_mixed_variant_name.argtypes = [ctypes.c_int]
        lib.gemm_mixed_variant_name.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.numel() and not x.is_cuda:
            raise TypeError("matrix tensors must live on the GPU")
        return x.data_ptr()
    return int(x)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int) -> None:
    if status != OK:
        raise GemmError(status, gemm_f32_status_string(status))


def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A x B on the library's default kernel; see gemm_f32.h."""
    lib = load_library()
    _check(lib.gemm_f32(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _stream(stream)))


def gemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A x B on a chosen rung (0..3) or diagnostic variant (16..)."""
    lib = load_library()
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    _check(lib.gemm_f32_variant(int(variant), M, N, K, _addr(A), lda, _addr(B), ldb,
                                _addr(C), ldc, _stream(stream)))


def gemm_f32_op(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = op(A) x op(B), op 'N' (as stored) or 'T' (stored transposed)."""
    lib = load_library()
    oa = OPS.get(op_a, op_a) if not isinstance(op_a, int) else op_a
    ob = OPS.get(op_b, op_b) if not isinstance(op_b, int) else op_b
    _check(lib.gemm_f32_op(int(oa), int(ob), M, N, K, _addr(A), lda, _addr(B), ldb,
                           _addr(C), ldc, _stream(stream)))


def gemm_f32_num_variants() -> int:
    return load_library().gemm_f32_num_variants()


def gemm_f32_num_diagnostic_variants() -> int:
    return load_library().gemm_f32_num_diagnostic_variants()


def gemm_f32_default_variant(M, N, K) -> int:
    """The diagnostic variant whose configuration gemm_f32 runs for M x N x K
    (-1 for invalid sizes); no device needed."""
    return int(load_library().gemm_f32_default_variant(M, N, K))


def gemm_f32_variant_name(variant: int) -> str | None:
    name = load_library().gemm_f32_variant_name(int(variant))
    return name.decode() if name is not None else None


def gemm_f32_status_string(status: int) -> str:
    return load_library().gemm_f32_status_string(int(status)).decode()


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.dtype != torch.float32:
        raise TypeError("matrices must be 2-D float32 tensors")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("matrices must be row-major (unit column stride)")
    return max(t.stride(0) if t.shape[0] > 1 else t.shape[1], t.shape[1], 1)


def gemm(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None,
         variant=None, stream=None, op_a="N", op_b="N") -> torch.Tensor:
    """Tensor form: returns ``out`` (allocated if None) = op(A) @ op(B).  A
    and B are the stored row-major tensors (with op 'T', A is K x M and B is
    N x K); views with a leading dimension (``stride(0)``) and a storage
    offset are passed through as they are.  ``variant`` selects a ladder
    rung and requires op 'N' for both factors."""
    M, K = A.shape if op_a in ("N", 0) else A.shape[::-1]
    K2, N = B.shape if op_b in ("N", 0) else B.shape[::-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    args = (M, N, K, A, _ld(A), B, _ld(B), out, _ld(out))
    if op_a not in ("N", 0) or op_b not in ("N", 0):
        if variant is not None:
            raise ValueError("transposed factors run on the default kernel only")
        gemm_f32_op(op_a, op_b, *args, stream=stream)
    elif variant is None:
        gemm_f32(*args, stream=stream)
    else:
        gemm_f32_variant(variant, *args, stream=stream)
    return out


def transpose_f32(rows, cols, src, ld_in, dst, ld_out, stream=None) -> None:
    """dst (cols x rows) = src (rows x cols) transposed; see gemm_f32.h."""
    lib = load_library()
    _check(lib.transpose_f32(rows, cols, _addr(src), ld_in, _addr(dst), ld_out, _stream(stream)))


def transpose_f32_variant(variant, rows, cols, src, ld_in, dst, ld_out, stream=None) -> None:
    lib = load_library()
    _check(lib.transpose_f32_variant(int(variant), rows, cols, _addr(src), ld_in, _addr(dst), ld_out,
                                     _stream(stream)))


def transpose_f32_num_variants() -> int:
    return load_library().transpose_f32_num_variants()


def transpose_f32_default_variant(rows, cols, ld_in, ld_out) -> int:
    """The variant transpose_f32 runs for these sizes (-1 for invalid ones)."""
    return int(load_library().transpose_f32_default_variant(rows, cols, ld_in, ld_out))


def transpose_f32_variant_name(variant: int) -> str | None:
    name = load_library().transpose_f32_variant_name(int(variant))
    return name.decode() if name is not None else None


def transpose(X: torch.Tensor, out: torch.Tensor | None = None, variant=None, stream=None) -> torch.Tensor:
    """Tensor form: returns ``out`` (allocated if None) = X^T for a 2-D
    float32 row-major CUDA tensor (views with a leading dimension allowed)."""
    rows, cols = X.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.float32, device=X.device)
    if tuple(out.shape) != (cols, rows):
        raise ValueError("out has the wrong shape")
    args = (rows, cols, X, _ld(X), out, _ld(out))
    if variant is None:
        transpose_f32(*args, stream=stream)
    else:
        transpose_f32_variant(variant, *args, stream=stream)
    return out


def gemm_f32_valu_probe(form, blocks, iters, out, stamps, stream=None) -> None:
    """The vector-ALU FMA loop of the library's measurement helper."""
    lib = load_library()
    _check(lib.gemm_f32_valu_probe(int(form), int(blocks), int(iters), _addr(out), _addr(stamps), _stream(stream)))


def gemm_f32_lds_probe(form, offsets, iters, out, stream=None) -> None:
    """The LDS read probe of the library's measurement helper (offsets: 64
    int32 on the device; out: 64 uint32 or int32 on the device)."""
    lib = load_library()
    _check(lib.gemm_f32_lds_probe(int(form), _addr(offsets), int(iters), _addr(out), _stream(stream)))


def gemm_f32_copy_probe(mode, blocks, iters, src, out, cycles, stream=None) -> None:
    """The copy-rate probe of the library's measurement helper."""
    lib = load_library()
    _check(lib.gemm_f32_copy_probe(int(mode), int(blocks), int(iters), _addr(src), _addr(out), _addr(cycles),
                                   _stream(stream)))


def gemm_f32_ksplit_timeline(M, N, K, A, lda, B, ldb, C, ldc, timeline, timeline_words, stream=None) -> None:
    """gemm_f32's k-split kernel with its per-wave timeline (measurement helper)."""
    lib = load_library()
    _check(lib.gemm_f32_ksplit_timeline(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _addr(timeline),
                                        int(timeline_words), _stream(stream)))


REDUCE_DEFAULT = 4


def reduce_sum_f32_workspace_size(variant: int, n: int) -> int:
    return load_library().reduce_sum_f32_workspace_size(int(variant), int(n))


def reduce_sum_f32(n, x, out, workspace, workspace_bytes, stream=None) -> None:
    """*out = sum of x[0 .. n-1] (device pointers); see gemm_f32.h."""
    lib = load_library()
    _check(lib.reduce_sum_f32(n, _addr(x), _addr(out), _addr(workspace), workspace_bytes, _stream(stream)))


def reduce_sum_f32_variant(variant, n, x, out, workspace, workspace_bytes, stream=None) -> None:
    lib = load_library()
    _check(lib.reduce_sum_f32_variant(int(variant), n, _addr(x), _addr(out), _addr(workspace),
                                      workspace_bytes, _stream(stream)))


def reduce_sum_f32_variant_noalloc(variant, n, x, out, stream=None) -> None:
    """reduce_sum_f32_variant with the partials in the library's fixed
    per-device scratch (no workspace, no allocation)."""
    lib = load_library()
    _check(lib.reduce_sum_f32_variant_noalloc(int(variant), n, _addr(x), _addr(out), _stream(stream)))


REDUCE_SCRATCH_BYTES = 1 << 20     # REDUCE_SUM_F32_SCRATCH_BYTES


def reduce_sum_f32_num_variants() -> int:
    return load_library().reduce_sum_f32_num_variants()


def reduce_sum_f32_variant_name(variant: int) -> str | None:
    name = load_library().reduce_sum_f32_variant_name(int(variant))
    return name.decode() if name is not None else None


def reduce_sum(x: torch.Tensor, variant=None, stream=None) -> torch.Tensor:
    """Tensor form: a one-element float32 CUDA tensor holding the sum of the
    contiguous float32 tensor x; the workspace is allocated with torch."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    n = x.numel()
    v = REDUCE_DEFAULT if variant is None else int(variant)
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws_bytes = reduce_sum_f32_workspace_size(v, n)
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=x.device)
    if variant is None:
        reduce_sum_f32(n, x, out, ws, ws_bytes, stream=stream)
    else:
        reduce_sum_f32_variant(v, n, x, out, ws, ws_bytes, stream=stream)
    return out


FORMATS = {"bf16": 0, "f16": 1}
_FORMAT_OF_DTYPE = {torch.bfloat16: 0, torch.float16: 1}


def _format(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt]
    return int(fmt)


def gemm_mixed(fmt, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C (binary32) = A x B for 16-bit A and B of format ``fmt`` ('bf16' or
    'f16'); leading dimensions in elements; see gemm_f32.h."""
    lib = load_library()
    _check(lib.gemm_mixed(_format(fmt), M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                          _stream(stream)))


def gemm_mixed_variant(variant, fmt, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    lib = load_library()
    _check(lib.gemm_mixed_variant(int(variant), _format(fmt), M, N, K, _addr(A), lda, _addr(B), ldb,
                                  _addr(C), ldc, _stream(stream)))


def gemm_mixed_op(op_a, op_b, fmt, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C (binary32) = op(A) x op(B) for 16-bit factors, op 'N' (as stored) or
    'T' (stored transposed: A is K x M, B is N x K); see gemm_f32.h."""
    lib = load_library()
    oa = OPS.get(op_a, op_a) if not isinstance(op_a, int) else op_a
    ob = OPS.get(op_b, op_b) if not isinstance(op_b, int) else op_b
    _check(lib.gemm_mixed_op(int(oa), int(ob), _format(fmt), M, N, K, _addr(A), lda, _addr(B), ldb,
                             _addr(C), ldc, _stream(stream)))


def gemm_mixed_num_variants() -> int:
    return load_library().gemm_mixed_num_variants()


def gemm_mixed_default_variant(M, N, K) -> int:
    """The configuration gemm_mixed runs for M x N x K (-1 for invalid
    sizes); no device needed."""
    return int(load_library().gemm_mixed_default_variant(M, N, K))


def gemm_mixed_variant_name(variant: int) -> str | None:
    name = load_library().gemm_mixed_variant_name(int(variant))
    return name.decode() if name is not None else None


def _ld16(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.dtype not in _FORMAT_OF_DTYPE:
        raise TypeError("16-bit factors must be 2-D bfloat16 or float16 tensors")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("matrices must be row-major (unit column stride)")
    return max(t.stride(0) if t.shape[0] > 1 else t.shape[1], t.shape[1], 1)


def gemm16(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None, variant=None,
           stream=None, op_a="N", op_b="N") -> torch.Tensor:
    """Tensor form: returns ``out`` (float32, allocated if None) = op(A) @
    op(B) for bfloat16 or float16 CUDA tensors of one dtype.  A and B are the
    stored row-major tensors (with op 'T', A is K x M and B is N x K); views
    with a leading dimension and a storage offset pass through.  ``variant``
    selects a tile configuration and requires op 'N' for both factors."""
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same 16-bit dtype")
    M, K = A.shape if op_a in ("N", 0) else A.shape[::-1]
    K2, N = B.shape if op_b in ("N", 0) else B.shape[::-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    args = (_FORMAT_OF_DTYPE[A.dtype], M, N, K, A, _ld16(A), B, _ld16(B), out, _ld(out))
    if op_a not in ("N", 0) or op_b not in ("N", 0):
        if variant is not None:
            raise ValueError("transposed factors run on the default kernels only")
        gemm_mixed_op(op_a, op_b, *args, stream=stream)
    elif variant is None:
        gemm_mixed(*args, stream=stream)
    else:
        gemm_mixed_variant(variant, *args, stream=stream)
    return out
