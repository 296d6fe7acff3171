"""The mixed-precision product with a transposed factor (gemm_mixed_op)
against the 16-bit oracle, and bit for bit against gemm_mixed on explicitly
transposed copies (the summation order does not depend on how a factor is
stored)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

OPS = [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")]
FORMATS = ["bf16", "f16"]
EDGE_SHAPES = [
    (1, 1, 1), (2, 3, 5), (7, 7, 7), (1, 300, 13), (300, 1, 13), (15, 17, 33), (63, 65, 127),
    (127, 129, 255), (257, 255, 1009), (33, 1009, 7), (511, 257, 65),
]


def stored(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


class OpProblem:
    def __init__(self, fmt, op_a, op_b, Ab, Bb, offset=0, pad=(0, 0, 0)):
        """Ab, Bb: the STORED 16-bit patterns (op 'T': A is K x M, B is N x K)."""
        self.fmt, self.op_a, self.op_b = fmt, op_a, op_b
        self.M, self.K = Ab.shape if op_a == "N" else Ab.shape[::-1]
        self.N = Bb.shape[1] if op_b == "N" else Bb.shape[0]
        self.A = inputs.padded16(Ab, max(Ab.shape[1] + pad[0], 1), offset, fmt)
        self.B = inputs.padded16(Bb, max(Bb.shape[1] + pad[1], 1), offset, fmt)
        self.ldc, self.offset = max(self.N + pad[2], 1), offset
        self.A_dev = torch.from_numpy(self.A.buf.view(np.int16)).cuda()
        self.B_dev = torch.from_numpy(self.B.buf.view(np.int16)).cuda()
        self.C_init = inputs.padded_output(self.M, self.N, self.ldc, offset)
        self.C_dev = torch.from_numpy(self.C_init.buf).cuda()

    def run(self, plain=False) -> inputs.Padded:
        self.C_dev.copy_(torch.from_numpy(self.C_init.buf))
        torch.cuda.synchronize()
        args = (self.fmt, self.M, self.N, self.K, self.A_dev.data_ptr() + 2 * self.A.offset, self.A.ld,
                self.B_dev.data_ptr() + 2 * self.B.offset, self.B.ld,
                self.C_dev.data_ptr() + 4 * self.offset, self.ldc)
        if plain:
            binding.gemm_mixed(*args)
        else:
            binding.gemm_mixed_op(self.op_a, self.op_b, *args)
        torch.cuda.synchronize()
        return inputs.Padded(self.C_dev.cpu().numpy(), self.M, self.N, self.ldc, self.offset)


def logical16(gen, fmt, M, N, K, dist):
    A = inputs.to16(inputs.random_matrix(gen, M, K, dist), fmt)
    B = inputs.to16(inputs.random_matrix(gen, K, N, dist), fmt)
    return A, B


def as_stored(op, X):
    return np.ascontiguousarray(X.T) if op == "T" else X


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_mixed_op_edge_shapes(ops, dist):
    """Every op pair on ragged shapes, aligned (vector loads, direct copies)
    and 2-byte-offset (element-wise loads), both formats: exact on integers,
    within 1e-5 S otherwise, padding untouched."""
    op_a, op_b = ops
    for fmt in FORMATS:
        for (M, N, K) in EDGE_SHAPES:
            for offset, pad in ((0, (0, 0, 0)), (1, (3, 5, 2))):
                gen = np.random.default_rng([M * 1_000_003 + N * 1009 + K, offset, len(fmt), len(op_a + op_b)])
                A, B = logical16(gen, fmt, M, N, K, dist)
                prob = OpProblem(fmt, op_a, op_b, as_stored(op_a, A), as_stored(op_b, B), offset, pad)
                say(f"mixed op {op_a}{op_b} {fmt} {dist} {M}x{N}x{K} offset={offset}")
                C = prob.run()
                Cref, S = oracle.gemm16(fmt, prob.A.view, prob.B.view, threads=8, op_a=op_a, op_b=op_b)
                if dist == "int":
                    check_exact(C.view, Cref, f"{op_a}{op_b} {fmt} {M}x{N}x{K}")
                else:
                    check_close(C.view, Cref, S, f"{op_a}{op_b} {fmt} {M}x{N}x{K}")
                check_padding_untouched(C)


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_op_bitwise_equal_to_plain(fmt):
    """For 128- and 256-wide tiles, ragged edges and a ghost k phase, and
    full tiles of the scheduled kernel with one, two and three phases, every
    op pair gives gemm_mixed's bits on the explicitly transposed factors."""
    for (M, N, K) in ((520, 530, 200), (1000, 1000, 1000), (4096, 4160, 264), (4096, 4096, 128), (4096, 4352, 64),
                      (4352, 4096, 192)):
        gen = np.random.default_rng([M, N, K, len(fmt)])
        A, B = logical16(gen, fmt, M, N, K, "uniform")
        plain = OpProblem(fmt, "N", "N", A, B).run(plain=True).view.copy()
        for op_a, op_b in OPS:
            say(f"mixed op bitwise {op_a}{op_b} {fmt} {M}x{N}x{K}")
            got = OpProblem(fmt, op_a, op_b, as_stored(op_a, A), as_stored(op_b, B)).run().view
            assert np.array_equal(got.view(np.uint32), plain.view(np.uint32)), (fmt, op_a, op_b, M, N, K)


@pytest.mark.parametrize("ops", [("T", "N"), ("N", "T")], ids=lambda o: o[0] + o[1])
def test_mixed_op_square8192_sampled(ops):
    """The backward-pass shapes at 8192^3: sampled entries against the oracle."""
    op_a, op_b = ops
    w = inputs.WORKLOADS["square8192"]
    fmt = "bf16"
    A32 = inputs.random_matrix(inputs.rng(w.index, 0), w.M, w.K, "uniform")
    B32 = inputs.random_matrix(inputs.rng(w.index, 1), w.K, w.N, "uniform")
    As = as_stored(op_a, inputs.to16(A32, fmt))
    Bs = as_stored(op_b, inputs.to16(B32, fmt))
    prob = OpProblem(fmt, op_a, op_b, As, Bs)
    say(f"mixed op {op_a}{op_b} square8192 sampled")
    C = prob.run()
    ii, jj = inputs.sample_pairs(w.M, w.N, 4096, inputs.rng(w.index, 4))
    c, s = oracle.gemm16_entries(fmt, prob.A.view, prob.B.view, ii, jj, op_a=op_a, op_b=op_b)
    check_close(C.view[ii, jj], c, s, f"{op_a}{op_b} square8192")
    check_padding_untouched(C)
    del prob
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_mixed_op_scheduled_exact(ops):
    """Full 256 x 256 tiles (the scheduled kernel for every op pair) with
    integer data: bit exact against the full oracle, both formats."""
    op_a, op_b = ops
    M, N, K = 4096, 4096, 192
    for fmt in FORMATS:
        gen = np.random.default_rng([M, N, K, len(fmt), len(op_a + op_b)])
        A, B = logical16(gen, fmt, M, N, K, "int")
        prob = OpProblem(fmt, op_a, op_b, as_stored(op_a, A), as_stored(op_b, B))
        say(f"mixed op scheduled {op_a}{op_b} {fmt} {M}x{N}x{K} int")
        C = prob.run()
        Cref, _ = oracle.gemm16(fmt, prob.A.view, prob.B.view, threads=16, op_a=op_a, op_b=op_b)
        check_exact(C.view, Cref, f"scheduled {op_a}{op_b} {fmt}")
        check_padding_untouched(C)
        del prob
        torch.cuda.empty_cache()


def test_mixed_op_tensor_form():
    gen = np.random.default_rng(11)
    A, B = logical16(gen, "bf16", 130, 150, 77, "uniform")
    At = torch.from_numpy(np.ascontiguousarray(A.T).view(np.int16)).cuda().view(torch.bfloat16)
    Bt = torch.from_numpy(np.ascontiguousarray(B.T).view(np.int16)).cuda().view(torch.bfloat16)
    C = binding.gemm16(At, Bt, op_a="T", op_b="T")
    torch.cuda.synchronize()
    Cref, S = oracle.gemm16("bf16", A, B)
    check_close(C.cpu().numpy(), Cref, S, "tensor form TT")


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_mixed_op_scheduled_edge_tiles(ops):
    """144 tiles of 256 x 256 with edge tiles (the scheduled kernel from 128
    such tiles) and integer data: bit exact against the full oracle and the
    bits of gemm_mixed on explicitly transposed copies.  Widths 3004 and
    2996 put a chunk across the end of an mn-contiguous factor's last row
    (zeros past it); with M (N) odd and even leading dimensions, A stored
    transposed (B as stored) runs the 8-wave kernel instead (on integer data
    every summation order gives the same exact bits).  K = 200: the last of
    four phases reaches past K (zeros there)."""
    op_a, op_b = ops
    for fmt in FORMATS:
        for (M, N, K, pad) in ((3000, 3000, 128, (0, 0, 0)), (3004, 2996, 192, (0, 0, 0)),
                               (3003, 2995, 64, (1, 1, 0)), (3000, 2996, 200, (0, 0, 0))):
            gen = np.random.default_rng([M, N, K, len(fmt), len(op_a + op_b), 5])
            A, B = logical16(gen, fmt, M, N, K, "int")
            prob = OpProblem(fmt, op_a, op_b, as_stored(op_a, A), as_stored(op_b, B), 0, pad)
            say(f"mixed op scheduled edges {op_a}{op_b} {fmt} {M}x{N}x{K} pad={pad} int")
            C = prob.run()
            check_padding_untouched(C)
            Cref, _ = oracle.gemm16(fmt, prob.A.view, prob.B.view, threads=16, op_a=op_a, op_b=op_b)
            check_exact(C.view, Cref, f"scheduled edges {op_a}{op_b} {fmt} {M}x{N}x{K}")
            plain = OpProblem(fmt, "N", "N", A, B).run(plain=True).view
            assert np.array_equal(C.view.view(np.uint32), plain.view(np.uint32)), (fmt, op_a, op_b, M, N, K)
