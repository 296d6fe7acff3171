"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Every check takes the loaded oracle library (a ctypes CDLL) and raises
AssertionError on a mismatch.  ``test_oracle.py`` runs them on the real
oracle; ``test_oracle_mutations.py`` runs them, in a subprocess, on copies of
the oracle with a planted mistake and expects at least one to fail.

None of these checks re-types the oracle's formula: they compare it with exact
integer arithmetic, closed forms, algebraic identities, an independent
binary64 library product, or the numbers the pages print
(``golden/pages_numbers.json``).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_numbers.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _ints(gen, rows, cols, lo=-2, hi=2):
    return gen.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)


def _py_product(A, B):
    """Exact integer product with Python ints (brute force)."""
    M, K = A.shape
    N = B.shape[1]
    a = [[int(x) for x in row] for row in A]
    b = [[int(x) for x in row] for row in B]
    C = [[0] * N for _ in range(M)]
    S = [[0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            c = s = 0
            for k in range(K):
                p = a[i][k] * b[k][j]
                c += p
                s += abs(p)
            C[i][j] = c
            S[i][j] = s
    return C, S


# ---------------------------------------------------------------- products --

def check_bruteforce_tiny(lib):
    """Integer inputs, every M, N, K in 1..9 and K = 0: exact equality with
    Python-int brute force, for C and for S."""
    gen = np.random.default_rng(101)
    sizes = [1, 2, 3, 5, 8, 9]
    for M, N, K in itertools.product(sizes, sizes, [0] + sizes):
        A = _ints(gen, M, K, -9, 9)
        B = _ints(gen, K, N, -9, 9)
        C, S = oracle.gemm(A, B, lib=lib)
        Ce, Se = _py_product(A, B)
        assert np.array_equal(C, np.array(Ce, dtype=np.float64).reshape(M, N)), (M, N, K)
        assert np.array_equal(S, np.array(Se, dtype=np.float64).reshape(M, N)), (M, N, K)


def check_bruteforce_tile_straddling(lib):
    """Integer inputs at sizes one below/above one and two tile edges for the
    tile sizes the kernels use: exact equality with int64 arithmetic."""
    gen = np.random.default_rng(102)
    for T in (16, 32, 64, 128):
        for (M, N, K) in ((T - 1, T + 1, 2 * T + 1), (T + 1, 2 * T - 1, T - 1),
                          (2 * T + 1, T - 1, T + 1)):
            A = _ints(gen, M, K)
            B = _ints(gen, K, N)
            C, S = oracle.gemm(A, B, threads=4, lib=lib)
            Ai, Bi = A.astype(np.int64), B.astype(np.int64)
            assert np.array_equal(C, (Ai @ Bi).astype(np.float64)), (T, M, N, K)
            assert np.array_equal(S, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)), (T, M, N, K)


def check_identity_and_zero(lib):
    """A I = A and I B = B exactly; A 0 and 0 B are +0 (not -0)."""
    gen = np.random.default_rng(103)
    A = (2 * gen.random((37, 23), dtype=np.float32) - 1).astype(np.float32)
    B = (2 * gen.random((23, 41), dtype=np.float32) - 1).astype(np.float32)
    C, _ = oracle.gemm(A, np.eye(23, dtype=np.float32), lib=lib)
    assert np.array_equal(C, A.astype(np.float64))
    C, _ = oracle.gemm(np.eye(23, dtype=np.float32), B, lib=lib)
    assert np.array_equal(C, B.astype(np.float64))
    C, S = oracle.gemm(A, np.zeros((23, 19), np.float32), lib=lib)
    assert np.all(C == 0) and not np.any(np.signbit(C)) and np.all(S == 0)
    C, S = oracle.gemm(np.zeros((11, 23), np.float32), B, lib=lib)
    assert np.all(C == 0) and not np.any(np.signbit(C)) and np.all(S == 0)
    # every product is -0 here; the sum starts from +0, so the result is +0
    C, _ = oracle.gemm(-np.ones((3, 23), np.float32), np.zeros((23, 4), np.float32), lib=lib)
    assert np.all(C == 0) and not np.any(np.signbit(C))
    # an empty sum (K = 0) is +0
    C, S = oracle.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32), lib=lib)
    assert np.all(C == 0) and not np.any(np.signbit(C)) and np.all(S == 0)


def check_closed_forms(lib):
    """All-ones gives K everywhere; A[i,k] = (i mod 7) - 3, B[k,j] = (j mod 5) - 2
    gives K ((i mod 7) - 3)((j mod 5) - 2)."""
    for (M, N, K) in ((33, 65, 17), (129, 31, 257)):
        C, S = oracle.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32), lib=lib)
        assert np.all(C == K) and np.all(S == K)
        i = np.arange(M)[:, None]
        j = np.arange(N)[None, :]
        A = np.broadcast_to((i % 7) - 3, (M, K)).astype(np.float32)
        B = np.broadcast_to((j % 5) - 2, (K, N)).astype(np.float32)
        C, S = oracle.gemm(np.ascontiguousarray(A), np.ascontiguousarray(B), lib=lib)
        assert np.array_equal(C, (K * ((i % 7) - 3) * ((j % 5) - 2)).astype(np.float64))
        assert np.array_equal(S, (K * np.abs((i % 7) - 3) * np.abs((j % 5) - 2)).astype(np.float64))


def check_library_float64(lib):
    """Against numpy's binary64 matmul on float inputs: within 1e-12 S."""
    gen = np.random.default_rng(104)
    for (M, N, K) in ((64, 48, 100), (17, 130, 257)):
        A = (2 * gen.random((M, K), dtype=np.float32) - 1).astype(np.float32)
        B = gen.standard_normal((K, N), dtype=np.float32)
        C, S = oracle.gemm(A, B, lib=lib)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        sref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.all(np.abs(C - ref) <= 1e-12 * sref)
        assert np.all(np.abs(S - sref) <= 1e-12 * sref)
        assert np.all(sref > 0)


def check_linearity_and_scaling(lib):
    """C(A, B1 + B2) = C(A, B1) + C(A, B2) to rounding (the sums B1 + B2 are
    exact in binary32 here), and C(2A, B) = 2 C(A, B) bit for bit."""
    gen = np.random.default_rng(105)
    M, N, K = 40, 50, 300
    A = (2 * gen.random((M, K), dtype=np.float32) - 1).astype(np.float32)
    B1 = (2 * gen.random((K, N), dtype=np.float32) - 1).astype(np.float32)
    B2 = (2 * gen.random((K, N), dtype=np.float32) - 1).astype(np.float32)
    Bs = (B1 + B2).astype(np.float32)
    assert np.array_equal(Bs.astype(np.float64), B1.astype(np.float64) + B2.astype(np.float64))
    C12, S12 = oracle.gemm(A, Bs, lib=lib)
    C1, S1 = oracle.gemm(A, B1, lib=lib)
    C2, S2 = oracle.gemm(A, B2, lib=lib)
    assert np.all(np.abs(C12 - C1 - C2) <= 1e-13 * (S1 + S2))
    C2A, S2A = oracle.gemm((2 * A).astype(np.float32), B1, lib=lib)
    assert np.array_equal(C2A, 2 * C1) and np.array_equal(S2A, 2 * S1)
    CA2, _ = oracle.gemm(A, (0.5 * B1).astype(np.float32), lib=lib)
    assert np.array_equal(CA2, 0.5 * C1)


def check_transpose_identity(lib):
    """(A B)^T = B^T A^T bit for bit: each entry sums the same products in the
    same k order, so a swapped operand or index shows up here."""
    gen = np.random.default_rng(106)
    A = gen.standard_normal((23, 57), dtype=np.float32)
    B = gen.standard_normal((57, 31), dtype=np.float32)
    C, S = oracle.gemm(A, B, lib=lib)
    Ct, St = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), lib=lib)
    assert np.array_equal(C.T, Ct) and np.array_equal(S.T, St)


def check_padded_views(lib):
    """Leading dimensions larger than the column count and a base offset of one
    float give the same bits as compact storage; NaN padding is never read."""
    gen = np.random.default_rng(107)
    M, N, K = 19, 29, 37
    A = gen.standard_normal((M, K), dtype=np.float32)
    B = gen.standard_normal((K, N), dtype=np.float32)
    C0, S0 = oracle.gemm(A, B, lib=lib)
    for lda, ldb, off in ((K + 3, N + 5, 1), (K + 8, N + 1, 3)):
        abuf = np.full(off + M * lda + 16, np.nan, np.float32)
        bbuf = np.full(off + K * ldb + 16, np.nan, np.float32)
        Av = abuf[off:off + M * lda].reshape(M, lda)[:, :K]
        Bv = bbuf[off:off + K * ldb].reshape(K, ldb)[:, :N]
        Av[:] = A
        Bv[:] = B
        C, S = oracle.gemm(Av, Bv, lib=lib)
        assert np.array_equal(C, C0) and np.array_equal(S, S0)


def check_entries_rows_threads(lib):
    """Selected entries, row bands and any thread count reproduce the full
    single-threaded product bit for bit."""
    gen = np.random.default_rng(108)
    M, N, K = 45, 38, 129
    A = gen.standard_normal((M, K), dtype=np.float32)
    B = gen.standard_normal((K, N), dtype=np.float32)
    C1, S1 = oracle.gemm(A, B, threads=1, lib=lib)
    C7, S7 = oracle.gemm(A, B, threads=7, lib=lib)
    assert np.array_equal(C1, C7) and np.array_equal(S1, S7)
    Cb, Sb = oracle.gemm(A, B, rows=(10, 21), threads=3, lib=lib)
    assert np.array_equal(Cb[10:21], C1[10:21]) and np.all(Cb[:10] == 0) and np.all(Cb[21:] == 0)
    ii = gen.integers(0, M, 200)
    jj = gen.integers(0, N, 200)
    c, s = oracle.gemm_entries(A, B, ii, jj, lib=lib)
    assert np.array_equal(c, C1[ii, jj]) and np.array_equal(s, S1[ii, jj])


def _padded_copy(X, extra, off):
    rows, cols = X.shape
    ld = cols + extra
    buf = np.full(off + rows * ld + 8, np.nan, np.float32)
    V = buf[off:off + rows * ld].reshape(rows, ld)[:, :cols]
    V[:] = X
    return V


def check_transposed_operands(lib):
    """op(A) x op(B) with A and/or B stored transposed (also in NaN-padded,
    offset storage) equals the plain product of the untransposed matrices bit
    for bit: the same products are summed in the same k order."""
    gen = np.random.default_rng(109)
    for (M, N, K) in ((23, 41, 57), (64, 9, 130), (1, 33, 7)):
        X = gen.standard_normal((M, K), dtype=np.float32)
        Y = (2 * gen.random((K, N), dtype=np.float32) - 1).astype(np.float32)
        C0, S0 = oracle.gemm(X, Y, lib=lib)
        Xt, Yt = np.ascontiguousarray(X.T), np.ascontiguousarray(Y.T)
        for (A, B, oa, ob) in ((Xt, Y, "T", "N"), (X, Yt, "N", "T"), (Xt, Yt, "T", "T"),
                               (_padded_copy(Xt, 3, 1), _padded_copy(Yt, 5, 2), "T", "T"),
                               (_padded_copy(Xt, 1, 0), Y, "T", "N")):
            C, S = oracle.gemm(A, B, op_a=oa, op_b=ob, threads=3, lib=lib)
            assert np.array_equal(C, C0) and np.array_equal(S, S0), (M, N, K, oa, ob)
            ii = gen.integers(0, M, 50)
            jj = gen.integers(0, N, 50)
            c, s2 = oracle.gemm_entries(A, B, ii, jj, op_a=oa, op_b=ob, lib=lib)
            assert np.array_equal(c, C0[ii, jj]) and np.array_equal(s2, S0[ii, jj])


def check_transposed_bruteforce(lib):
    """Integer inputs, tiny shapes, every op combination: exact equality with
    Python-int brute force on the transposes built element by element."""
    gen = np.random.default_rng(110)
    for (M, N, K) in ((2, 3, 4), (5, 1, 3), (3, 7, 2), (6, 4, 9)):
        for oa in ("N", "T"):
            for ob in ("N", "T"):
                A = _ints(gen, M, K, -7, 7) if oa == "N" else _ints(gen, K, M, -7, 7)
                B = _ints(gen, K, N, -7, 7) if ob == "N" else _ints(gen, N, K, -7, 7)
                opA = [[int(A[i][k]) if oa == "N" else int(A[k][i]) for k in range(K)] for i in range(M)]
                opB = [[int(B[k][j]) if ob == "N" else int(B[j][k]) for j in range(N)] for k in range(K)]
                Ce, Se = _py_product(np.array(opA, dtype=np.float32).reshape(M, K),
                                     np.array(opB, dtype=np.float32).reshape(K, N))
                C, S = oracle.gemm(A, B, op_a=oa, op_b=ob, lib=lib)
                assert np.array_equal(C, np.array(Ce, dtype=np.float64).reshape(M, N)), (oa, ob, M, N, K)
                assert np.array_equal(S, np.array(Se, dtype=np.float64).reshape(M, N)), (oa, ob, M, N, K)


# ------------------------------------------------------ traffic bookkeeping --

def check_naive_intensity(lib):
    """One thread per output reads one A and one B float per multiply-add:
    0.25 FLOP/B, the pages' naive figure, for square and ragged shapes."""
    g = _golden()["naive_intensity"]["flop_per_byte"]
    for (M, N, K) in ((8, 8, 8), (5, 7, 3), (16, 4, 9)):
        t = oracle.tiled_traffic(M, N, K, 1, 1, 1, lib=lib)
        flop = 2 * t["macs_useful"]
        byts = 4 * (t["a_loads"] + t["b_loads"])
        assert flop / byts == g and t["a_ghosts"] == 0 and t["b_ghosts"] == 0
        assert t["macs_useful"] == M * N * K


def check_tiled_intensity_and_traffic(lib):
    """Square N, tile T dividing N: 8NT bytes and 2N T^2 FLOP per block,
    intensity T/4 (4 at 16, 8 at 32), 2N/T floats read per output, and the
    traffic ratios 1/16 and 1/32 -- all as printed on the pages."""
    gold = _golden()
    ai = gold["tiled_intensity"]["flop_per_byte_by_tile"]
    gain = gold["tiled_intensity"]["gain_over_naive_by_tile"]
    ratio = gold["traffic_per_output"]["ratio_by_tile"]
    naive = gold["naive_intensity"]["flop_per_byte"]
    for T in (16, 32):
        N = 4 * T
        t = oracle.tiled_traffic(N, N, N, T, T, T, lib=lib)
        blocks = t["tiles"]
        assert blocks == (N // T) ** 2 and t["phases"] == N // T
        bytes_per_block = 4 * (t["a_loads"] + t["b_loads"]) / blocks
        flop_per_block = 2 * t["macs_useful"] / blocks
        assert bytes_per_block == 8 * N * T
        assert flop_per_block == 2 * N * T * T
        assert flop_per_block / bytes_per_block == ai[str(T)]
        assert (flop_per_block / bytes_per_block) / naive == gain[str(T)]
        per_output = (t["a_loads"] + t["b_loads"]) / (N * N)
        assert per_output == 2 * N / T
        assert per_output / (2 * N) == ratio[str(T)]


def check_tiled_traffic_ragged(lib):
    """Ragged shapes: reads are M K ceil(N/BN) + K N ceil(M/BM), ghosts fill
    the rest of every staged tile, useful multiply-adds are M N K, and the
    per-phase staging of a square T tile is the pages' 2 T^2 floats."""
    for (M, N, K, BM, BN, BK) in ((37, 45, 29, 16, 16, 16), (33, 17, 65, 32, 16, 8),
                                  (100, 100, 100, 64, 32, 16), (5, 6, 7, 8, 8, 8)):
        t = oracle.tiled_traffic(M, N, K, BM, BN, BK, lib=lib)
        tm, tn, ph = -(-M // BM), -(-N // BN), -(-K // BK)
        assert t["tiles"] == tm * tn and t["phases"] == ph
        assert t["a_loads"] == M * K * tn and t["b_loads"] == K * N * tm
        assert t["a_loads"] + t["a_ghosts"] == tm * tn * ph * BM * BK
        assert t["b_loads"] + t["b_ghosts"] == tm * tn * ph * BK * BN
        assert t["macs_issued"] == tm * tn * ph * BM * BN * BK
        assert t["macs_useful"] == M * N * K
    smem = _golden()["shared_memory_per_block"]
    for T in (16, 32, 64):
        t = oracle.tiled_traffic(T, T, T, T, T, T, lib=lib)
        staged_bytes = 4 * (t["a_loads"] + t["a_ghosts"] + t["b_loads"] + t["b_ghosts"])
        assert staged_bytes == smem["kb_by_tile"][str(T)] * 1024
        assert smem["limit_kb"] * 1024 // staged_bytes == smem["blocks_by_tile"][str(T)]


def check_naive_roofline_context(lib):
    """The pages' A100 context: bandwidth times the naive intensity gives the
    0.375 TFLOPS bound, about 1.9 percent of 19.5 TFLOPS."""
    g = _golden()["naive_roofline_a100"]
    t = oracle.tiled_traffic(4, 4, 4, 1, 1, 1, lib=lib)
    ai = 2 * t["macs_useful"] / (4 * (t["a_loads"] + t["b_loads"]))
    bound = g["bandwidth_tb_s"] * ai
    assert math.isclose(bound, g["bound_tflops"], rel_tol=1e-12)
    assert round(100 * bound / g["peak_tflops"], 1) == g["fraction_percent"]


# ------------------------------------------------------------- bank model --

def check_bank_model(lib):
    """gcd(S, 32)-way conflicts for the pages' strides; column reads of a
    [32][32] tile are 32-way, of a [32][33] tile conflict free; an XOR-swizzled
    [32][32] tile is conflict free by rows and by columns; in the tiled product
    the B-tile row read is spread and the A-tile read is a broadcast."""
    g = _golden()["bank_conflicts"]
    lanes = np.arange(32, dtype=np.int64)
    for S, deg in g["degree_by_stride"].items():
        assert oracle.bank_conflict_degree(lanes * int(S), g["banks"], lib=lib) == deg
        assert deg == math.gcd(int(S), 32)
    c = 5
    assert oracle.bank_conflict_degree(lanes * 32 + c, lib=lib) == g["transpose_column_read_32x32"]
    assert oracle.bank_conflict_degree(lanes * 33 + c, lib=lib) == g["transpose_column_read_32x33"]
    for y in range(32):   # row y written by lanes x = 0..31 at column x ^ y
        assert oracle.bank_conflict_degree(y * 32 + (lanes ^ y), lib=lib) == g["transpose_xor_swizzle_row_and_column"]
    for x in range(32):   # column x read by lanes y = 0..31 at column y ^ x ... of row y
        assert oracle.bank_conflict_degree(lanes * 32 + (x ^ lanes), lib=lib) == g["transpose_xor_swizzle_row_and_column"]
    k, ty = 7, 3
    assert oracle.bank_conflict_degree(k * 32 + lanes, lib=lib) == g["tiled_product_reads"]       # Bs[k][tx]
    assert oracle.bank_conflict_degree(np.full(32, ty * 32 + k), lib=lib) == g["tiled_product_reads"]  # As[ty][k]


# --------------------------------------------------------------- transpose --

def check_transpose(lib):
    """The transpose against brute force on tiny shapes, numpy's transpose,
    and the involution (transposing twice gives the input back bit for bit),
    in padded, offset storage whose padding must stay untouched."""
    gen = np.random.default_rng(111)
    for rows, cols in ((1, 1), (1, 7), (5, 1), (3, 4), (4, 3)):
        X = gen.standard_normal((rows, cols), dtype=np.float32)
        T = oracle.transpose(X, lib=lib)
        for r in range(rows):
            for c in range(cols):
                assert T[c, r] == X[r, c], (rows, cols, r, c)
    for rows, cols in ((37, 53), (64, 33), (129, 257)):
        X = gen.standard_normal((rows, cols), dtype=np.float32)
        T = oracle.transpose(X, lib=lib)
        assert np.array_equal(T, X.T)
        assert np.array_equal(oracle.transpose(T, lib=lib), X)
        Xp = _padded_copy(X, 3, 1)
        buf = np.full(1 + cols * (rows + 5) + 8, 7.5, np.float32)
        Tv = buf[1:1 + cols * (rows + 5)].reshape(cols, rows + 5)[:, :rows]
        oracle.transpose_into(Xp, Tv, lib=lib)
        assert np.array_equal(Tv, X.T)
        mask = np.ones(buf.shape, bool)
        for c in range(cols):
            mask[1 + c * (rows + 5): 1 + c * (rows + 5) + rows] = False
        assert np.all(buf[mask] == 7.5)


def check_sector_model(lib):
    """The first page's coalescing numbers: 32 lanes of 4-byte floats touch
    128 bytes of 32-byte sectors when aligned, 160 bytes when shifted by one
    float, and 1024 bytes when the lanes are 32 bytes apart."""
    g = _golden()["coalescing_sectors"]
    sb, n, w = g["sector_bytes"], g["lanes"], g["float_bytes"]
    lanes = np.arange(n, dtype=np.int64)
    assert oracle.sectors_touched(lanes * w, w, sb, lib=lib) * sb == g["aligned_bytes"]
    assert oracle.sectors_touched(lanes * w + w, w, sb, lib=lib) * sb == g["shifted_one_float_bytes"]
    assert oracle.sectors_touched(lanes * 32, w, sb, lib=lib) * sb == g["stride_32_bytes"]
    assert oracle.sectors_touched(lanes * 64, w, sb, lib=lib) * sb == g["stride_32_bytes"]
    # a repeated address is one access, a straddling one counts both sectors
    assert oracle.sectors_touched(np.zeros(n, np.int64), w, sb, lib=lib) == 1
    assert oracle.sectors_touched(np.array([30], np.int64), 4, sb, lib=lib) == 2


# --------------------------------------------------------------- reduction --

def check_sum(lib):
    """The binary64 sum: exact on integers (closed form and int64 sums), on
    the empty array +0, and within n 2^-53 sum|x| of the exact sum of floats
    (math.fsum); sum|x| likewise."""
    gen = np.random.default_rng(112)
    s, a = oracle.reduce_sum(np.zeros(0, np.float32), lib=lib)
    assert s == 0.0 and not math.copysign(1.0, s) < 0 and a == 0.0
    n = 100_000
    ramp = np.arange(1, n + 1, dtype=np.float32)
    s, a = oracle.reduce_sum(ramp, lib=lib)
    assert s == n * (n + 1) // 2 and a == s
    for size in (1, 7, 1000, 65537):
        xi = gen.integers(-3, 4, size)
        s, a = oracle.reduce_sum(xi.astype(np.float32), lib=lib)
        assert s == float(xi.sum()) and a == float(np.abs(xi).sum())
    for size in (17, 4096, 300001):
        x = gen.standard_normal(size, dtype=np.float32)
        s, a = oracle.reduce_sum(x, lib=lib)
        exact = math.fsum(x.astype(np.float64).tolist())
        assert abs(s - exact) <= size * 2.0**-53 * a
        assert abs(a - math.fsum(np.abs(x).astype(np.float64).tolist())) <= size * 2.0**-53 * a
        assert a > 0


def check_tree_bookkeeping(lib):
    """The page's tree counts: 8 steps and 255 additions for 256 elements in
    both versions, and 47 (version 0) against 12 (version 1) warp steps with
    32-thread warps; a tree over N values always does N - 1 additions."""
    g = _golden()["reduction"]
    for version, key in ((0, "warp_steps_version0"), (1, "warp_steps_version1")):
        t = oracle.tree_counts(g["block"], g["warp"], version, lib=lib)
        assert t["steps"] == g["steps"] and t["adds"] == g["adds"] and t["warp_steps"] == g[key]
    for b in (2, 8, 64, 1024):
        for version in (0, 1):
            t = oracle.tree_counts(b, 64, version, lib=lib)
            assert t["adds"] == b - 1 and t["steps"] == int(math.log2(b))


def check_multipass(lib):
    """2^24 values, 256 per block: 65,536 -> 256 -> 1, three launches."""
    g = _golden()["reduction"]
    k, sizes = oracle.reduce_passes(g["multipass_n"], g["multipass_per_block"], lib=lib)
    assert k == g["multipass_launches"] and sizes == g["multipass_sizes"]
    assert oracle.reduce_passes(1, 256, lib=lib)[0] == 0
    assert oracle.reduce_passes(257, 256, lib=lib) == (2, [257, 2, 1])

# ------------------------------------------- 16-bit inputs, fp32 result --

def _widen16(bits, fmt):
    """binary32 values of 16-bit patterns by numpy's own decoding: binary16
    through numpy's float16, bfloat16 as the upper half of a binary32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if fmt == "f16":
        with np.errstate(invalid="ignore"):
            return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _encode_exact16(x, fmt):
    """Patterns of values that are exact in the format (checked)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "f16":
        b = x.astype(np.float16).view(np.uint16)
    else:
        w = x.view(np.uint32)
        assert np.all((w & 0xFFFF) == 0)
        b = (w >> 16).astype(np.uint16)
    assert np.array_equal(_widen16(b, fmt), x)
    return b


def _finite16(gen, shape, fmt):
    """Random finite 16-bit patterns (every sign, exponent and fraction)."""
    b = gen.integers(0, 65536, size=shape).astype(np.uint16)
    exp_all_ones = (b & 0x7F80) == 0x7F80 if fmt == "bf16" else (b & 0x7C00) == 0x7C00
    b[exp_all_ones] &= np.uint16(0xBFFF)         # clear the top exponent bit
    return b


def check_decode16_all_patterns(lib):
    """Every one of the 65,536 patterns of both formats decodes to numpy's
    value for it (NaN to NaN, each zero with its sign), and a few values the
    formats' definitions fix: 1, the largest finite and the smallest
    subnormal of each."""
    b = np.arange(65536, dtype=np.uint16)
    for fmt in ("f16", "bf16"):
        got = oracle.decode16(fmt, b, lib=lib)
        with np.errstate(invalid="ignore"):
            ref = _widen16(b, fmt).astype(np.float64)
        assert np.array_equal(got, ref, equal_nan=True), fmt
        assert np.array_equal(np.signbit(got), np.signbit(ref)), fmt
    known = {("f16", 0x3C00): 1.0, ("f16", 0x7BFF): 65504.0, ("f16", 0x0001): 2.0**-24,
             ("f16", 0x0400): 2.0**-14, ("f16", 0xC000): -2.0,
             ("bf16", 0x3F80): 1.0, ("bf16", 0x7F7F): (2 - 2.0**-7) * 2.0**127,
             ("bf16", 0x0001): 2.0**-133, ("bf16", 0x0080): 2.0**-126, ("bf16", 0xC000): -2.0}
    for (fmt, bits), v in known.items():
        assert oracle.decode16(fmt, np.array([bits], np.uint16), lib=lib)[0] == v, (fmt, hex(bits))


def check_gemm16_equals_fp32_oracle(lib):
    """Random finite patterns of both formats, at tile-straddling shapes and in
    padded offset views: the 16-bit product equals the fp32 oracle on the same
    values widened to binary32, bit for bit, for C and S; row bands, thread
    counts and single entries agree with the full product."""
    gen = np.random.default_rng(120)
    for fmt in ("bf16", "f16"):
        for (M, N, K) in ((1, 1, 1), (17, 33, 65), (64, 31, 129), (33, 64, 0)):
            A = _finite16(gen, (M, K), fmt)
            B = _finite16(gen, (K, N), fmt)
            C, S = oracle.gemm16(fmt, A, B, lib=lib)
            C32, S32 = oracle.gemm(_widen16(A, fmt), _widen16(B, fmt), lib=lib)
            assert np.array_equal(C, C32) and np.array_equal(S, S32), (fmt, M, N, K)
            # padded views with an odd element offset
            Ap = np.full(3 + M * (K + 5) + 7, 0x7E00, np.uint16)
            Av = Ap[3:3 + M * (K + 5)].reshape(M, K + 5)[:, :K]
            Av[:, :] = A
            Bp = np.full(1 + K * (N + 2) + 7, 0x7E00, np.uint16)
            Bv = Bp[1:1 + K * (N + 2)].reshape(K, N + 2)[:, :N] if K else B
            if K:
                Bv[:, :] = B
            Cv, Sv = oracle.gemm16(fmt, Av, Bv, threads=3, lib=lib)
            assert np.array_equal(Cv, C) and np.array_equal(Sv, S), (fmt, M, N, K)
            if M > 2 and N:
                Cb, _ = oracle.gemm16(fmt, A, B, rows=(1, M - 1), lib=lib)
                assert np.array_equal(Cb[1:M - 1], C[1:M - 1]) and np.all(Cb[0] == 0)
                ii = gen.integers(0, M, 20)
                jj = gen.integers(0, N, 20)
                c, sv = oracle.gemm16_entries(fmt, Av, Bv, ii, jj, lib=lib)
                assert np.array_equal(c, C[ii, jj]) and np.array_equal(sv, S[ii, jj])


def check_gemm16_bruteforce(lib):
    """Integers -9..9 (exact in both formats), every M, N in {1, 2, 3, 5, 8}
    and K in {0, 1, 2, 3, 5, 8}: exact equality with Python-int brute force."""
    gen = np.random.default_rng(121)
    sizes = [1, 2, 3, 5, 8]
    for fmt in ("bf16", "f16"):
        for M, N, K in itertools.product(sizes, sizes, [0] + sizes):
            A = _ints(gen, M, K, -9, 9)
            B = _ints(gen, K, N, -9, 9)
            C, S = oracle.gemm16(fmt, _encode_exact16(A, fmt), _encode_exact16(B, fmt), lib=lib)
            Ce, Se = _py_product(A, B)
            assert np.array_equal(C, np.array(Ce, dtype=np.float64).reshape(M, N)), (fmt, M, N, K)
            assert np.array_equal(S, np.array(Se, dtype=np.float64).reshape(M, N)), (fmt, M, N, K)


def check_gemm16_extremes(lib):
    """The formats' range ends inside the product: binary16's largest finite
    value 65504 squared and summed K times, its smallest subnormal 2^-24
    squared (2^-48 per term, far below binary16 but exact in the sum);
    bfloat16's largest finite times 2^-126 and its smallest subnormal 2^-133
    times 2^100; all-ones gives K; signs of mixed terms."""
    K = 37
    for fmt, big, tiny, one, exp in (("f16", 0x7BFF, 0x0001, 0x3C00, None),
                                     ("bf16", 0x7F7F, 0x0001, 0x3F80, (0x0080, 0x71 << 7))):
        A = np.full((2, K), one, np.uint16)
        B = np.full((K, 3), one, np.uint16)
        C, S = oracle.gemm16(fmt, A, B, lib=lib)
        assert np.all(C == K) and np.all(S == K)
        if fmt == "f16":
            A[0, :] = big
            B[:, 0] = big
            A[1, :] = tiny
            B[:, 1] = tiny
            C, _ = oracle.gemm16(fmt, A, B, lib=lib)
            assert C[0, 0] == K * 65504.0**2 and C[1, 1] == K * 2.0**-48 and C[0, 1] == K * 65504.0 * 2.0**-24
        else:
            A[0, :] = big
            B[:, 0] = exp[0]                      # 2^-126
            A[1, :] = tiny                        # 2^-133
            B[:, 1] = exp[1]                      # 2^(0x71 - 127) = 2^-14
            C, _ = oracle.gemm16(fmt, A, B, lib=lib)
            assert C[0, 0] == K * (2 - 2.0**-7) * 2.0 and C[1, 1] == K * 2.0**-147
        A = np.full((1, 4), one, np.uint16)
        A[0, 1] |= np.uint16(0x8000)              # -1
        B = np.full((4, 1), one, np.uint16)
        B[3, 0] |= np.uint16(0x8000)
        C, S = oracle.gemm16(fmt, A, B, lib=lib)
        assert C[0, 0] == 0.0 and S[0, 0] == 4.0     # 1 - 1 + 1 - 1


def check_gemm16_transposed_operands(lib):
    """op(A) and op(B) for every op pair and both formats: bit equality with
    the plain 16-bit product on explicitly transposed copies (C and S), in
    padded odd-offset views, for full products, row bands and entries; and
    exact integer brute force for the logical factors."""
    gen = np.random.default_rng(122)
    for fmt in ("bf16", "f16"):
        for (M, N, K) in ((1, 1, 1), (17, 33, 65), (64, 31, 129)):
            A = _finite16(gen, (M, K), fmt)
            B = _finite16(gen, (K, N), fmt)
            C, S = oracle.gemm16(fmt, A, B, lib=lib)
            for op_a, op_b in (("T", "N"), ("N", "T"), ("T", "T")):
                As = np.ascontiguousarray(A.T) if op_a == "T" else A
                Bs = np.ascontiguousarray(B.T) if op_b == "T" else B
                Ap = np.full(3 + As.shape[0] * (As.shape[1] + 5) + 7, 0x7E00, np.uint16)
                Av = Ap[3:3 + As.shape[0] * (As.shape[1] + 5)].reshape(As.shape[0], As.shape[1] + 5)[:, :As.shape[1]]
                Av[:, :] = As
                Co, So = oracle.gemm16(fmt, Av, Bs, threads=3, lib=lib, op_a=op_a, op_b=op_b)
                assert np.array_equal(Co, C) and np.array_equal(So, S), (fmt, M, N, K, op_a, op_b)
                ii = gen.integers(0, M, 15)
                jj = gen.integers(0, N, 15)
                c, sv = oracle.gemm16_entries(fmt, Av, Bs, ii, jj, lib=lib, op_a=op_a, op_b=op_b)
                assert np.array_equal(c, C[ii, jj]) and np.array_equal(sv, S[ii, jj]), (fmt, op_a, op_b)
    for fmt in ("bf16", "f16"):
        for (M, N, K) in ((2, 3, 5), (5, 1, 8), (8, 5, 3)):
            Ai = _ints(gen, M, K, -9, 9)
            Bi = _ints(gen, K, N, -9, 9)
            Ce, _ = _py_product(Ai, Bi)
            for op_a, op_b in (("T", "N"), ("N", "T"), ("T", "T")):
                As = np.ascontiguousarray(Ai.T) if op_a == "T" else Ai
                Bs = np.ascontiguousarray(Bi.T) if op_b == "T" else Bi
                Co, _ = oracle.gemm16(fmt, _encode_exact16(As, fmt), _encode_exact16(Bs, fmt), lib=lib,
                                      op_a=op_a, op_b=op_b)
                assert np.array_equal(Co, np.array(Ce, dtype=np.float64).reshape(M, N)), (fmt, op_a, op_b)


ALL_CHECKS = [
    check_bruteforce_tiny, check_bruteforce_tile_straddling, check_identity_and_zero,
    check_closed_forms, check_library_float64, check_linearity_and_scaling,
    check_transpose_identity, check_padded_views, check_entries_rows_threads,
    check_transposed_operands, check_transposed_bruteforce,
    check_naive_intensity, check_tiled_intensity_and_traffic, check_tiled_traffic_ragged,
    check_naive_roofline_context, check_bank_model, check_transpose, check_sector_model,
    check_sum, check_tree_bookkeeping, check_multipass,
    check_decode16_all_patterns, check_gemm16_equals_fp32_oracle, check_gemm16_bruteforce,
    check_gemm16_extremes, check_gemm16_transposed_operands,
]


def run_all(lib):
    """Runs every check; returns the names of those that failed."""
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk(lib)
        except AssertionError:
            failed.append(chk.__name__)
    return failed


if __name__ == "__main__":      # used by the mutation test in a subprocess
    import sys
    lib = oracle.load(sys.argv[1])
    bad = run_all(lib)
    print("FAILED:" + ",".join(bad))
    sys.exit(3 if bad else 0)
