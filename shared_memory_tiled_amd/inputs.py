"""Seeded synthetic inputs for the fp32 GEMM workloads.

This module holds no part of the product's arithmetic: it only draws random
matrices, lays them out in padded row-major buffers and picks output entries
to check.  Both sides of every parity test (the HIP library and the CPU
oracle) take their operands from here; nothing else is shared between them.

Workloads (the shapes the pages' tiled kernel is exercised on, extended to
general sizes with leading dimensions):

    square256      M=N=K=256, uniform[-1,1); integer variant in {-2..2}
    square1000     M=N=K=1000 (not a multiple of 16/32/64/128), uniform[-1,1)
    square4096     M=N=K=4096, standard normal
    rect8192x4096x2048_padded
                   M=8192, N=4096, K=2048, lda=2056, ldb=ldc=4104, every view
                   starting one float into its allocation (not 16-byte
                   aligned), uniform[-1,1)
    square8192     M=N=K=8192, uniform[-1,1); checked on a seeded sample of
                   4096 entries plus edge entries

"uniform[-1,1)" is 2u - 1 with u drawn as binary32 on the 2^-24 grid, which
is exact in binary32 and never reaches +1.

The mixed-precision product takes the same workloads in a 16-bit format
(bfloat16 or binary16): the binary32 data above rounded to the format,
nearest-even, and held as uint16 bit patterns; pads and guards hold the
format's quiet NaN.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202

# The pad and guard words around every operand; A and B padding holds NaN so
# that a stray read poisons the result, C padding holds this quiet-NaN bit
# pattern, which must survive the call untouched.
C_SENTINEL_BITS = np.uint32(0x7FC0DEAD)
GUARD_WORDS = 64


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    offset: int          # floats between the allocation start and the view
    dist: str            # "uniform", "normal"
    index: int           # seed index
    sampled: bool        # checked on a sample of entries instead of in full


WORKLOADS = {
    w.name: w for w in (
        Workload("square256", 256, 256, 256, 256, 256, 256, 0, "uniform", 0, False),
        Workload("square1000", 1000, 1000, 1000, 1000, 1000, 1000, 0, "uniform", 1, False),
        Workload("square4096", 4096, 4096, 4096, 4096, 4096, 4096, 0, "normal", 2, True),
        Workload("rect8192x4096x2048_padded", 8192, 4096, 2048, 2056, 4104, 4104, 1,
                 "uniform", 3, True),
        Workload("square8192", 8192, 8192, 8192, 8192, 8192, 8192, 0, "uniform", 4, True),
    )
}


def rng(index: int, stream: int) -> np.random.Generator:
    """Generator for workload ``index``; stream 0 = A, 1 = B, 2/3 = integer A/B,
    4 = sample positions, larger streams are free for tests."""
    return np.random.default_rng([SEED_BASE + index, stream])


def random_matrix(gen: np.random.Generator, rows: int, cols: int, dist: str) -> np.ndarray:
    """A dense rows x cols binary32 matrix with the named distribution."""
    if dist == "uniform":
        u = gen.random((rows, cols), dtype=np.float32)
        return (np.float32(2.0) * u - np.float32(1.0)).astype(np.float32)
    if dist == "normal":
        return gen.standard_normal((rows, cols), dtype=np.float32)
    if dist == "int":          # small integers -2..2, exactly representable
        return gen.integers(-2, 3, size=(rows, cols)).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


@dataclass
class Padded:
    """A rows x cols matrix inside a larger 1-D buffer: element (r, c) sits at
    buf[offset + r*ld + c]; everything else in buf is padding or guard."""
    buf: np.ndarray
    rows: int
    cols: int
    ld: int
    offset: int

    @property
    def view(self) -> np.ndarray:
        n = self.rows * self.ld
        return self.buf[self.offset:self.offset + n].reshape(self.rows, self.ld)[:, :self.cols] \
            if self.rows > 0 else self.buf[self.offset:self.offset].reshape(0, self.cols)


def padded(dense: np.ndarray, ld: int, offset: int = 0, fill=np.nan,
           guard: int = GUARD_WORDS) -> Padded:
    """Copy ``dense`` into a padded buffer whose pad and guard words hold ``fill``."""
    rows, cols = dense.shape
    if ld < max(cols, 1):
        raise ValueError("leading dimension smaller than the column count")
    buf = np.empty(offset + rows * ld + guard, dtype=np.float32)
    buf[:] = fill
    p = Padded(buf, rows, cols, ld, offset)
    if rows:
        p.view[:, :] = dense
    return p


def padded_output(rows: int, cols: int, ld: int, offset: int = 0,
                  guard: int = GUARD_WORDS) -> Padded:
    """An output buffer filled entirely with the C sentinel pattern."""
    buf = np.empty(offset + rows * ld + guard, dtype=np.float32)
    buf.view(np.uint32)[:] = C_SENTINEL_BITS
    return Padded(buf, rows, cols, ld, offset)


def operands(w: Workload, dist: str | None = None, offset: int | None = None):
    """(A, B) as Padded host buffers for workload ``w``.  ``dist="int"``
    gives the integer-valued variant (separate seed streams)."""
    d = dist or w.dist
    off = w.offset if offset is None else offset
    sa, sb = (2, 3) if d == "int" else (0, 1)
    A = random_matrix(rng(w.index, sa), w.M, w.K, d)
    B = random_matrix(rng(w.index, sb), w.K, w.N, d)
    return padded(A, w.lda, off), padded(B, w.ldb, off)


def sample_pairs(M: int, N: int, count: int, gen: np.random.Generator,
                 tiles=(16, 32, 64, 128, 256)):
    """``count`` distinct (i, j) drawn uniformly without replacement, plus the
    four corners and, for every tile edge in ``tiles``, one entry from the
    last partial tile row and column.  Returns (ii, jj) int64 arrays."""
    if M == 0 or N == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    total = M * N
    flat = gen.choice(total, size=min(count, total), replace=False).astype(np.int64)
    ii = list(flat // N)
    jj = list(flat % N)
    extra = {(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)}
    for t in tiles:
        r0 = (M - 1) // t * t
        c0 = (N - 1) // t * t
        extra.add((r0, int(gen.integers(0, N))))
        extra.add((int(gen.integers(0, M)), c0))
        extra.add((M - 1, c0))
        extra.add((r0, N - 1))
    have = set(zip(ii, jj))
    for (i, j) in sorted(extra):
        if (i, j) not in have:
            ii.append(i)
            jj.append(j)
    return np.asarray(ii, dtype=np.int64), np.asarray(jj, dtype=np.int64)


# 16-bit formats: name -> quiet-NaN pattern used for padding.
NAN16 = {"bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


def to16(x: np.ndarray, fmt: str) -> np.ndarray:
    """Bit patterns (uint16) of the binary32 array ``x`` rounded to ``fmt``,
    nearest-even.  binary16 uses numpy's conversion; for bfloat16 the lower
    half of each binary32 pattern is rounded away (finite inputs only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        if not np.all(np.isfinite(x)):
            raise ValueError("bfloat16 rounding here takes finite values only")
        bits = x.view(np.uint32).astype(np.uint64)
        return ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    raise ValueError(f"unknown 16-bit format {fmt!r}")


def padded16(bits: np.ndarray, ld: int, offset: int, fmt: str, guard: int = GUARD_WORDS) -> Padded:
    """Copy the uint16 matrix ``bits`` into a padded uint16 buffer whose pad
    and guard elements hold the format's quiet NaN."""
    rows, cols = bits.shape
    if ld < max(cols, 1):
        raise ValueError("leading dimension smaller than the column count")
    buf = np.empty(offset + rows * ld + guard, dtype=np.uint16)
    buf[:] = NAN16[fmt]
    p = Padded(buf, rows, cols, ld, offset)
    if rows:
        p.view[:, :] = bits
    return p


def operands16(w: Workload, fmt: str, dist: str | None = None, offset: int | None = None):
    """(A, B) of workload ``w`` rounded to ``fmt``, as padded uint16 host
    buffers with the workload's leading dimensions (in elements), and the
    binary32 data they were rounded from (dense)."""
    d = dist or w.dist
    off = w.offset if offset is None else offset
    sa, sb = (2, 3) if d == "int" else (0, 1)
    A32 = random_matrix(rng(w.index, sa), w.M, w.K, d)
    B32 = random_matrix(rng(w.index, sb), w.K, w.N, d)
    return (padded16(to16(A32, fmt), w.lda, off, fmt), padded16(to16(B32, fmt), w.ldb, off, fmt),
            A32, B32)
