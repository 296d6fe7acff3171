"""Products with a transposed factor (gemm_f32_op) against the oracle, and
bit for bit against the plain product on explicitly transposed copies."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

OPS = [("T", "N"), ("N", "T"), ("T", "T")]
EDGE_SHAPES = [
    (1, 1, 1), (2, 3, 5), (7, 7, 7), (1, 300, 13), (300, 1, 13), (15, 17, 33),
    (63, 65, 127), (127, 129, 255), (257, 255, 1009), (33, 1009, 7), (511, 257, 33),
]


def stored_shape(op, rows, cols):
    """Shape of the stored matrix whose op() is rows x cols."""
    return (rows, cols) if op == "N" else (cols, rows)


class OpProblem:
    def __init__(self, op_a, op_b, M, N, K, dist, gen, offset=0, pad=(0, 0, 0)):
        self.op_a, self.op_b, self.M, self.N, self.K = op_a, op_b, M, N, K
        ar, ac = stored_shape(op_a, M, K)
        br, bc = stored_shape(op_b, K, N)
        self.A = inputs.padded(inputs.random_matrix(gen, ar, ac, dist), ac + pad[0], offset)
        self.B = inputs.padded(inputs.random_matrix(gen, br, bc, dist), bc + pad[1], offset)
        self.ldc, self.offset = N + pad[2], offset
        self.A_dev = torch.from_numpy(self.A.buf).cuda()
        self.B_dev = torch.from_numpy(self.B.buf).cuda()
        self.C_init = inputs.padded_output(M, N, self.ldc, offset)
        self.C_dev = torch.from_numpy(self.C_init.buf).cuda()

    def run(self):
        self.C_dev.copy_(torch.from_numpy(self.C_init.buf))
        binding.gemm_f32_op(self.op_a, self.op_b, self.M, self.N, self.K,
                            self.A_dev.data_ptr() + 4 * self.A.offset, self.A.ld,
                            self.B_dev.data_ptr() + 4 * self.B.offset, self.B.ld,
                            self.C_dev.data_ptr() + 4 * self.offset, self.ldc)
        torch.cuda.synchronize()
        return inputs.Padded(self.C_dev.cpu().numpy(), self.M, self.N, self.ldc, self.offset)


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_op_edge_shapes(ops, dist):
    op_a, op_b = ops
    for (M, N, K) in EDGE_SHAPES:
        for offset in (0, 1):
            gen = np.random.default_rng([M * 1_000_003 + N * 1009 + K, offset, len(op_a + op_b)])
            prob = OpProblem(op_a, op_b, M, N, K, dist, gen, offset, pad=(3 * offset, 5 * offset, 2))
            Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
            say(f"op={op_a}{op_b} dist={dist} shape={(M, N, K)} offset={offset}")
            C = prob.run()
            check_padding_untouched(C)
            what = f"{op_a}{op_b} {dist} {(M, N, K)} offset {offset}"
            if dist == "int":
                check_exact(C.view, Cref, what)
            else:
                check_close(C.view, Cref, S, what)


def transposed_copy(t: torch.Tensor) -> torch.Tensor:
    return t.t().contiguous()


# One shape per tile configuration the default path picks (16x16 and 32x32
# small tiles with k groups split over the waves, 64x64 split over four wave
# groups with 32- and 16-deep phases, 128x128 register-staged, 128x128 and
# 256x256 on four scheduled waves, 256x256 on eight waves with a ghost k
# phase, and with ragged edges as well).
SAME_BITS_SHAPES = [(300, 200, 130), (500, 400, 257), (1000, 1000, 380), (2100, 2050, 300), (3840, 2048, 100),
                    (2048, 2048, 96), (4096, 4096, 512), (4096, 4096, 515), (8193, 8190, 99)]


@pytest.mark.parametrize("shape", SAME_BITS_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_op_same_bits_as_plain_product(shape):
    """The k order depends only on M, N, K, so every op pair must give the
    same bits as gemm_f32 on explicitly transposed copies."""
    M, N, K = shape
    gen = torch.Generator(device="cuda").manual_seed(M + N + K)
    X = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
    Y = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
    say(f"same bits {shape} NN")
    ref = binding.gemm(X, Y)
    for op_a, op_b in OPS:
        A = transposed_copy(X) if op_a == "T" else X
        B = transposed_copy(Y) if op_b == "T" else Y
        say(f"same bits {shape} {op_a}{op_b}")
        out = binding.gemm(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} {shape} differs from the plain product"


@functools.lru_cache(maxsize=None)
def large_case(name, op_a, op_b):
    w = inputs.WORKLOADS[name]
    gen = inputs.rng(w.index, 10 + 2 * (op_a == "T") + (op_b == "T"))
    prob = OpProblem(op_a, op_b, w.M, w.N, w.K, w.dist, gen)
    return w, prob


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("name", ["square4096", "square8192"])
def test_op_large_sampled(name, ops):
    op_a, op_b = ops
    say(f"generating {name} op={op_a}{op_b}")
    w, prob = large_case(name, op_a, op_b)
    ii, jj = inputs.sample_pairs(w.M, w.N, 4096, inputs.rng(w.index, 4))
    cref, sref = oracle.gemm_entries(prob.A.view, prob.B.view, ii, jj, op_a=op_a, op_b=op_b)
    say(f"running {name} op={op_a}{op_b}")
    C = prob.run()
    check_padding_untouched(C)
    check_close(C.view[ii, jj], cref, sref, f"{name} {op_a}{op_b}")
    assert np.all(np.isfinite(C.view))
