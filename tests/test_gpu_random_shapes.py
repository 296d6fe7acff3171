"""Seeded random problems through the default entry points (gemm_f32_op and
gemm_mixed_op, which cover gemm_f32 and gemm_mixed for op N, N) against the
oracle: random sizes (so every configuration the size-based choice can make
is reached), random op pairs, view offsets and padded leading dimensions.
Integer data bit exact, uniform data within 1e-5 S, padding untouched.  The
large-tile cases (256 x 256 tiles, the scheduled 16-bit kernel) are checked
on sampled entries."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

SEED = 20261202


def log_uniform(gen, lo, hi):
    return int(round(np.exp(gen.uniform(np.log(lo), np.log(hi)))))


def small_cases(n, max_work, stream):
    gen = np.random.default_rng([SEED, stream])
    out = []
    while len(out) < n:
        M, N, K = log_uniform(gen, 1, 3000), log_uniform(gen, 1, 3000), log_uniform(gen, 1, 1500)
        if M * N * K > max_work:
            continue
        ops = ("N" if gen.random() < 0.5 else "T", "N" if gen.random() < 0.5 else "T")
        offset = int(gen.integers(0, 2))
        pad = tuple(int(x) for x in gen.integers(0, 8, size=3))
        dist = "int" if len(out) % 2 == 0 else "uniform"
        out.append((M, N, K, ops, offset, pad, dist))
    return out


def large_cases(n, stream, multiple_of=1):
    gen = np.random.default_rng([SEED, stream])
    out = []
    for i in range(n):
        M = 4096 + multiple_of * int(gen.integers(0, 300 // multiple_of + 1))
        N = 4096 + multiple_of * int(gen.integers(0, 300 // multiple_of + 1))
        K = 64 * int(gen.integers(1, 7)) if multiple_of > 1 else int(gen.integers(32, 400))
        ops = ("N" if gen.random() < 0.5 else "T", "N" if gen.random() < 0.5 else "T")
        out.append((M, N, K, ops, 0, (0, 0, 0), "uniform"))
    return out


def stored(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


class Problem:
    """Padded stored factors (NaN padding), a sentinel-filled C; fmt None for
    binary32 factors, else "bf16" or "f16"."""

    def __init__(self, fmt, M, N, K, ops, offset, pad, dist, gen):
        self.fmt, self.M, self.N, self.K, self.ops, self.offset = fmt, M, N, K, ops, offset
        ar, ac = stored(ops[0], M, K)
        br, bc = stored(ops[1], K, N)
        A32 = inputs.random_matrix(gen, ar, ac, dist)
        B32 = inputs.random_matrix(gen, br, bc, dist)
        if fmt is None:
            self.A = inputs.padded(A32, max(ac + pad[0], 1), offset)
            self.B = inputs.padded(B32, max(bc + pad[1], 1), offset)
            self.A_dev = torch.from_numpy(self.A.buf).cuda()
            self.B_dev = torch.from_numpy(self.B.buf).cuda()
            self.esize = 4
        else:
            self.A = inputs.padded16(inputs.to16(A32, fmt), max(ac + pad[0], 1), offset, fmt)
            self.B = inputs.padded16(inputs.to16(B32, fmt), max(bc + pad[1], 1), offset, fmt)
            self.A_dev = torch.from_numpy(self.A.buf.view(np.int16)).cuda()
            self.B_dev = torch.from_numpy(self.B.buf.view(np.int16)).cuda()
            self.esize = 2
        self.ldc = max(N + pad[2], 1)
        self.C_init = inputs.padded_output(M, N, self.ldc, offset)
        self.C_dev = torch.from_numpy(self.C_init.buf).cuda()

    def run(self) -> inputs.Padded:
        e = self.esize
        args = (self.M, self.N, self.K, self.A_dev.data_ptr() + e * self.A.offset, self.A.ld,
                self.B_dev.data_ptr() + e * self.B.offset, self.B.ld,
                self.C_dev.data_ptr() + 4 * self.offset, self.ldc)
        if self.fmt is None:
            binding.gemm_f32_op(self.ops[0], self.ops[1], *args)
        else:
            binding.gemm_mixed_op(self.ops[0], self.ops[1], self.fmt, *args)
        torch.cuda.synchronize()
        return inputs.Padded(self.C_dev.cpu().numpy(), self.M, self.N, self.ldc, self.offset)

    def oracle_full(self):
        if self.fmt is None:
            return oracle.gemm(self.A.view, self.B.view, threads=16, op_a=self.ops[0], op_b=self.ops[1])
        return oracle.gemm16(self.fmt, self.A.view, self.B.view, threads=16, op_a=self.ops[0], op_b=self.ops[1])

    def oracle_entries(self, ii, jj):
        if self.fmt is None:
            return oracle.gemm_entries(self.A.view, self.B.view, ii, jj, op_a=self.ops[0], op_b=self.ops[1])
        return oracle.gemm16_entries(self.fmt, self.A.view, self.B.view, ii, jj, op_a=self.ops[0], op_b=self.ops[1])


def describe(fmt, case):
    M, N, K, ops, offset, pad, dist = case
    return f"{fmt or 'f32'} {ops[0]}{ops[1]} {M}x{N}x{K} offset={offset} pad={pad} {dist}"


def check_full(fmt, case, index):
    M, N, K, ops, offset, pad, dist = case
    prob = Problem(fmt, M, N, K, ops, offset, pad, dist, np.random.default_rng([SEED, 100, index]))
    say(f"random case {index}: {describe(fmt, case)}")
    C = prob.run()
    Cref, S = prob.oracle_full()
    if dist == "int":
        check_exact(C.view, Cref, describe(fmt, case))
    else:
        check_close(C.view, Cref, S, describe(fmt, case))
    check_padding_untouched(C)


def check_sampled(fmt, case, index):
    M, N, K, ops, offset, pad, dist = case
    prob = Problem(fmt, M, N, K, ops, offset, pad, dist, np.random.default_rng([SEED, 200, index]))
    say(f"random large case {index}: {describe(fmt, case)}")
    C = prob.run()
    ii, jj = inputs.sample_pairs(M, N, 2048, np.random.default_rng([SEED, 300, index]))
    c, s = prob.oracle_entries(ii, jj)
    check_close(C.view[ii, jj], c, s, describe(fmt, case))
    check_padding_untouched(C)
    del prob
    torch.cuda.empty_cache()


def test_random_fp32_small():
    for i, case in enumerate(small_cases(48, 6e7, 1)):
        check_full(None, case, i)


def test_random_fp32_large_tiles():
    for i, case in enumerate(large_cases(4, 2)):
        check_sampled(None, case, i)


def test_random_mixed_small():
    gen = np.random.default_rng([SEED, 3])
    for i, case in enumerate(small_cases(40, 6e7, 4)):
        check_full("bf16" if gen.random() < 0.5 else "f16", case, 1000 + i)


def test_random_mixed_large_tiles():
    """Multiples of 256 and 64 (the scheduled kernel) and ragged ones (its
    fallback), every op pair at random."""
    cases = large_cases(3, 5, multiple_of=256) + large_cases(2, 6)
    for i, case in enumerate(cases):
        check_sampled("bf16" if i % 2 == 0 else "f16", case, 2000 + i)
