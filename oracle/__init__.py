"""CPU oracle for the dense fp32 product C = A x B (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``gemm_oracle.c`` (plain C, binary64 accumulation);
this module only compiles it with gcc, loads it with ctypes and marshals
numpy arrays.  See the C file's header for what each function follows on the
pages ("03 CUDA Shared Memory: Tiling, Bank Conflicts, and Reduction" and the
PMPP chapter 5 notes "메모리 계층과 데이터 지역성").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_SOURCES = [_SRC, os.path.join(_HERE, "transpose_oracle.c"), os.path.join(_HERE, "reduce_oracle.c"),
            os.path.join(_HERE, "gemm16_oracle.c")]
_LIB = os.path.join(_HERE, "libgemm_oracle.so")

_i64 = ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_hp = ctypes.POINTER(ctypes.c_uint16)

_lib = None


def build(src: str | None = None, out: str = _LIB, replace: dict | None = None) -> str:
    """Compile the oracle sources into one shared library (gcc, strict IEEE
    arithmetic).  ``replace`` maps a source's base name to another file to
    compile in its place (``src`` is the same for gemm_oracle.c).  The
    library is written under a temporary name and renamed into place, so
    concurrent builders never expose a partly written file."""
    replace = dict(replace or {})
    if src is not None:
        replace["gemm_oracle.c"] = src
    sources = [replace.get(os.path.basename(s), s) for s in _SOURCES]
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-shared", "-fPIC", "-pthread", "-o", tmp, *sources, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) the oracle library; returns the CDLL."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    stale = path is None and os.path.exists(p) and \
        max(os.path.getmtime(src) for src in _SOURCES) > os.path.getmtime(p)
    if not os.path.exists(p) or stale:
        build(out=p)
    lib = ctypes.CDLL(p)
    lib.oracle_gemm_op_rows.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _fp, _i64,
                                        _fp, _i64, _dp, _i64, _dp, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_gemm_op_rows.restype = ctypes.c_int
    lib.oracle_gemm_op_entries.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _fp, _i64,
                                           _fp, _i64, _i64, _ip, _ip, _dp, _dp]
    lib.oracle_gemm_op_entries.restype = ctypes.c_int
    lib.oracle_gemm_rows.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64,
                                     _dp, _i64, _dp, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64,
                                _dp, _i64, _dp, _i64, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [_i64, _i64, _i64, _fp, _i64, _fp, _i64,
                                        _i64, _ip, _ip, _dp, _dp]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    lib.oracle_tiled_traffic.argtypes = [_i64] * 6 + [_ip]
    lib.oracle_tiled_traffic.restype = ctypes.c_int
    lib.oracle_bank_conflict_degree.argtypes = [_i64, _ip, _i64]
    lib.oracle_bank_conflict_degree.restype = _i64
    lib.oracle_transpose.argtypes = [_i64, _i64, _fp, _i64, _fp, _i64]
    lib.oracle_transpose.restype = ctypes.c_int
    lib.oracle_sectors_touched.argtypes = [_i64, _ip, _i64, _i64]
    lib.oracle_sectors_touched.restype = _i64
    lib.oracle_sum.argtypes = [_i64, _fp, _dp, _dp]
    lib.oracle_sum.restype = ctypes.c_int
    lib.oracle_tree_counts.argtypes = [_i64, _i64, ctypes.c_int, _ip]
    lib.oracle_tree_counts.restype = ctypes.c_int
    lib.oracle_reduce_passes.argtypes = [_i64, _i64, _ip, _i64]
    lib.oracle_reduce_passes.restype = _i64
    lib.oracle_decode16_array.argtypes = [ctypes.c_int, _i64, _hp, _dp]
    lib.oracle_decode16_array.restype = ctypes.c_int
    lib.oracle_gemm16_rows.argtypes = [ctypes.c_int, _i64, _i64, _i64, _hp, _i64, _hp, _i64,
                                       _dp, _i64, _dp, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_gemm16_rows.restype = ctypes.c_int
    lib.oracle_gemm16_op_rows.argtypes = [ctypes.c_int, ctypes.c_int] + lib.oracle_gemm16_rows.argtypes
    lib.oracle_gemm16_op_rows.restype = ctypes.c_int
    lib.oracle_gemm16_entries.argtypes = [ctypes.c_int, _i64, _i64, _i64, _hp, _i64, _hp, _i64,
                                          _i64, _ip, _ip, _dp, _dp]
    lib.oracle_gemm16_entries.restype = ctypes.c_int
    lib.oracle_gemm16_op_entries.argtypes = [ctypes.c_int, ctypes.c_int] + lib.oracle_gemm16_entries.argtypes
    lib.oracle_gemm16_op_entries.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _matrix_arg(X: np.ndarray):
    """(pointer, leading dimension) of a 2-D float32 row-major (possibly
    padded) view; the view's rows may be spaced wider than its columns."""
    if X.dtype != np.float32 or X.ndim != 2:
        raise TypeError("oracle operands must be 2-D float32 arrays")
    if X.size == 0:
        return ctypes.cast(ctypes.c_void_p(X.ctypes.data), _fp), max(X.shape[1], 1)
    if X.shape[1] > 1 and X.strides[1] != 4:
        raise ValueError("oracle operands need unit column stride")
    if X.strides[0] % 4:
        raise ValueError("row stride must be a whole number of floats")
    ld = X.strides[0] // 4 if X.shape[0] > 1 else max(X.shape[1], 1)
    ld = max(ld, X.shape[1], 1)
    ptr = X.ctypes.data_as(_fp)
    return ptr, ld


def _op(op) -> int:
    if op in (0, "N", "n"):
        return 0
    if op in (1, "T", "t"):
        return 1
    raise ValueError(f"op must be 'N' or 'T', not {op!r}")


def _shapes(A, B, op_a, op_b):
    M, K = A.shape if op_a == 0 else A.shape[::-1]
    K2, N = B.shape if op_b == 0 else B.shape[::-1]
    if K != K2:
        raise ValueError("inner dimensions differ")
    return M, N, K


def gemm(A: np.ndarray, B: np.ndarray, threads: int = 1, rows=None, lib=None,
         op_a="N", op_b="N"):
    """Returns (C, S): binary64 product op(A) x op(B) and sum_k |op(A)_ik op(B)_kj|.

    A and B are the STORED matrices: with op_a = 'T', A is K x M and op(A)
    is its transpose; with op_b = 'T', B is N x K.  ``rows=(r0, r1)``
    computes only that band of rows (the other rows stay zero)."""
    lib = lib or load()
    oa, ob = _op(op_a), _op(op_b)
    M, N, K = _shapes(A, B, oa, ob)
    C = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    pa, lda = _matrix_arg(A)
    pb, ldb = _matrix_arg(B)
    r0, r1 = (0, M) if rows is None else rows
    if oa == 0 and ob == 0:           # the plain entry point, as pinned
        rc = lib.oracle_gemm_rows(M, N, K, pa, lda, pb, ldb,
                                  C.ctypes.data_as(_dp), max(N, 1),
                                  S.ctypes.data_as(_dp), max(N, 1),
                                  r0, r1, int(threads))
    else:
        rc = lib.oracle_gemm_op_rows(oa, ob, M, N, K, pa, lda, pb, ldb,
                                     C.ctypes.data_as(_dp), max(N, 1),
                                     S.ctypes.data_as(_dp), max(N, 1),
                                     r0, r1, int(threads))
    if rc != 0:
        raise ValueError(f"oracle product rejected its arguments (rc={rc})")
    return C, S


def gemm_entries(A: np.ndarray, B: np.ndarray, ii, jj, lib=None, op_a="N", op_b="N"):
    """Returns (c, s) for the entries (ii[t], jj[t]) of op(A) x op(B) only."""
    lib = lib or load()
    oa, ob = _op(op_a), _op(op_b)
    M, N, K = _shapes(A, B, oa, ob)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D of equal length")
    c = np.zeros(ii.shape[0], dtype=np.float64)
    s = np.zeros(ii.shape[0], dtype=np.float64)
    pa, lda = _matrix_arg(A)
    pb, ldb = _matrix_arg(B)
    args = (M, N, K, pa, lda, pb, ldb, ii.shape[0], ii.ctypes.data_as(_ip), jj.ctypes.data_as(_ip),
            c.ctypes.data_as(_dp), s.ctypes.data_as(_dp))
    rc = lib.oracle_gemm_entries(*args) if oa == 0 and ob == 0 else \
        lib.oracle_gemm_op_entries(oa, ob, *args)
    if rc != 0:
        raise ValueError(f"oracle entries rejected their arguments (rc={rc})")
    return c, s


TRAFFIC_FIELDS = ("a_loads", "b_loads", "a_ghosts", "b_ghosts",
                  "macs_issued", "macs_useful", "tiles", "phases")


def tiled_traffic(M, N, K, BM, BN, BK, lib=None) -> dict:
    """Brute-force count of global reads / ghost slots / multiply-adds of the
    tiled phase loop with BM x BN output tiles and BK-deep phases."""
    lib = lib or load()
    out = (ctypes.c_int64 * 8)()
    rc = lib.oracle_tiled_traffic(M, N, K, BM, BN, BK, out)
    if rc != 0:
        raise ValueError("oracle_tiled_traffic rejected its arguments")
    return dict(zip(TRAFFIC_FIELDS, list(out)))


def bank_conflict_degree(word_addrs, banks: int = 32, lib=None) -> int:
    """Conflict degree of one shared-memory access (4-byte word addresses)."""
    lib = lib or load()
    w = np.ascontiguousarray(word_addrs, dtype=np.int64)
    return int(lib.oracle_bank_conflict_degree(w.shape[0], w.ctypes.data_as(_ip), banks))


def transpose_into(X: np.ndarray, out: np.ndarray, lib=None) -> None:
    """Writes the transpose of the 2-D float32 view X into the 2-D view out
    (shape X.shape[::-1]); words of out's buffer outside the view are left as
    they are."""
    lib = lib or load()
    rows, cols = X.shape
    if out.shape != (cols, rows) or out.dtype != np.float32:
        raise ValueError("out must be a float32 view of shape X.shape[::-1]")
    px, ldx = _matrix_arg(X)
    po, ldo = _matrix_arg(out)
    rc = lib.oracle_transpose(rows, cols, px, ldx, po, ldo)
    if rc != 0:
        raise ValueError("oracle_transpose rejected its arguments")


def transpose(X: np.ndarray, lib=None) -> np.ndarray:
    """The transpose of the 2-D float32 view X as a new compact array."""
    out = np.zeros(X.shape[::-1], dtype=np.float32)
    transpose_into(X, out, lib=lib)
    return out


def sectors_touched(byte_addrs, width: int, sector_bytes: int = 32, lib=None) -> int:
    """Distinct aligned sectors touched when lane l reads `width` bytes at
    byte address byte_addrs[l]."""
    lib = lib or load()
    a = np.ascontiguousarray(byte_addrs, dtype=np.int64)
    n = int(lib.oracle_sectors_touched(a.shape[0], a.ctypes.data_as(_ip), width, sector_bytes))
    if n < 0:
        raise ValueError("oracle_sectors_touched rejected its arguments")
    return n


def reduce_sum(x: np.ndarray, lib=None):
    """(sum, sum of |x|) of a 1-D float32 array, in binary64, index order."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    s = ctypes.c_double()
    a = ctypes.c_double()
    ptr = x.ctypes.data_as(_fp) if x.size else ctypes.cast(ctypes.c_void_p(0), _fp)
    rc = lib.oracle_sum(x.size, ptr, ctypes.byref(s), ctypes.byref(a))
    if rc != 0:
        raise ValueError("oracle_sum rejected its arguments")
    return s.value, a.value


def tree_counts(block: int, warp: int, version: int, lib=None) -> dict:
    """Steps, additions and active-warp steps of one block's tree reduction."""
    lib = lib or load()
    out = (ctypes.c_int64 * 3)()
    if lib.oracle_tree_counts(block, warp, version, out) != 0:
        raise ValueError("oracle_tree_counts rejected its arguments")
    return {"steps": out[0], "adds": out[1], "warp_steps": out[2]}


def reduce_passes(n: int, per_block: int, lib=None):
    """(launches, sizes after each launch) of the multi-pass scheme."""
    lib = lib or load()
    sizes = (ctypes.c_int64 * 64)()
    k = int(lib.oracle_reduce_passes(n, per_block, sizes, 64))
    if k < 0:
        raise ValueError("oracle_reduce_passes rejected its arguments")
    return k, [sizes[i] for i in range(k + 1)]


FORMATS16 = {"bf16": 0, "f16": 1}


def _fmt16(fmt) -> int:
    if fmt in FORMATS16:
        return FORMATS16[fmt]
    if fmt in (0, 1):
        return int(fmt)
    raise ValueError(f"16-bit format must be 'bf16' or 'f16', not {fmt!r}")


def _matrix16_arg(X: np.ndarray):
    """(pointer, leading dimension) of a 2-D uint16 row-major (possibly
    padded) view holding 16-bit patterns."""
    if X.dtype != np.uint16 or X.ndim != 2:
        raise TypeError("16-bit oracle operands must be 2-D uint16 arrays of bit patterns")
    if X.size == 0:
        return ctypes.cast(ctypes.c_void_p(X.ctypes.data), _hp), max(X.shape[1], 1)
    if X.shape[1] > 1 and X.strides[1] != 2:
        raise ValueError("oracle operands need unit column stride")
    if X.strides[0] % 2:
        raise ValueError("row stride must be a whole number of elements")
    ld = X.strides[0] // 2 if X.shape[0] > 1 else max(X.shape[1], 1)
    return X.ctypes.data_as(_hp), max(ld, X.shape[1], 1)


def decode16(fmt, bits, lib=None) -> np.ndarray:
    """Values (binary64) of an array of 16-bit patterns."""
    lib = lib or load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(b.shape, dtype=np.float64)
    if b.size and lib.oracle_decode16_array(_fmt16(fmt), b.size, b.ctypes.data_as(_hp),
                                            out.ctypes.data_as(_dp)) != 0:
        raise ValueError("oracle_decode16_array rejected its arguments")
    return out


def gemm16(fmt, A: np.ndarray, B: np.ndarray, threads: int = 1, rows=None, lib=None,
           op_a="N", op_b="N"):
    """Returns (C, S) in binary64 for op(A) x op(B), 16-bit factors given as
    uint16 bit patterns of format ``fmt`` ('bf16' or 'f16').  A and B are
    the STORED matrices (with op 'T', A is K x M and B is N x K)."""
    lib = lib or load()
    oa, ob = _op(op_a), _op(op_b)
    M, N, K = _shapes(A, B, oa, ob)
    C = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    pa, lda = _matrix16_arg(A)
    pb, ldb = _matrix16_arg(B)
    r0, r1 = (0, M) if rows is None else rows
    args = (_fmt16(fmt), M, N, K, pa, lda, pb, ldb,
            C.ctypes.data_as(_dp), max(N, 1), S.ctypes.data_as(_dp), max(N, 1), r0, r1, int(threads))
    rc = lib.oracle_gemm16_rows(*args) if oa == 0 and ob == 0 else lib.oracle_gemm16_op_rows(oa, ob, *args)
    if rc != 0:
        raise ValueError(f"oracle 16-bit product rejected its arguments (rc={rc})")
    return C, S


def gemm16_entries(fmt, A: np.ndarray, B: np.ndarray, ii, jj, lib=None, op_a="N", op_b="N"):
    """Returns (c, s) for the entries (ii[t], jj[t]) of the 16-bit product
    op(A) x op(B)."""
    lib = lib or load()
    oa, ob = _op(op_a), _op(op_b)
    M, N, K = _shapes(A, B, oa, ob)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D of equal length")
    c = np.zeros(ii.shape[0], dtype=np.float64)
    s = np.zeros(ii.shape[0], dtype=np.float64)
    pa, lda = _matrix16_arg(A)
    pb, ldb = _matrix16_arg(B)
    args = (_fmt16(fmt), M, N, K, pa, lda, pb, ldb, ii.shape[0], ii.ctypes.data_as(_ip),
            jj.ctypes.data_as(_ip), c.ctypes.data_as(_dp), s.ctypes.data_as(_dp))
    rc = lib.oracle_gemm16_entries(*args) if oa == 0 and ob == 0 else lib.oracle_gemm16_op_entries(oa, ob, *args)
    if rc != 0:
        raise ValueError(f"oracle 16-bit entries rejected their arguments (rc={rc})")
    return c, s
