"""The four-wave scheduled fp32 kernel on 256 x 256 and 128 x 128 tiles,
which gemm_f32 and gemm_f32_op run when K, M and N are multiples of 4 (the
256 x 256 form when its tiles fill their rounds of 256 workgroups to 95 %,
else the 128 x 128 form when there are at least 128 such tiles, unless the
k-split 64 x 64 tiles win the cost model; edge tiles run whole and store only
what lies inside C, and a last phase that reaches past K copies zeros there).

Checked against the oracle (every entry on short-K problems, sampled
entries on longer ones; exact on integer inputs) for all four op pairs, on
aligned and on padded, dword-offset operands, and bit for bit against the
kernel of the same tile size that other shapes use (eight-wave 256 x 256,
register-staged 128 x 128) on explicitly transposed copies: all sum every
entry's k terms in the same order."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# kernel -> (its configuration, the same-tile kernel it must match bit for bit)
KERNELS = {
    "tile256": ("mfma256x256_bk32_w2x2_sched", "mfma256x256_bk32_w2x4_direct"),
    "tile128": ("mfma128x128_bk32_w2x2_sched", "mfma128x128_bk16_w2x2"),
}


def variant_number(name):
    for d in range(binding.gemm_f32_num_diagnostic_variants()):
        if binding.gemm_f32_variant_name(binding.DIAGNOSTIC_BASE + d) == name:
            return binding.DIAGNOSTIC_BASE + d
    raise KeyError(name)


def stored_shape(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


class Problem:
    """op(A) x op(B) on padded device buffers (pad words NaN, C sentinels)."""

    def __init__(self, op_a, op_b, M, N, K, dist, seed, offset=0, pad=(0, 0, 0)):
        self.op_a, self.op_b, self.M, self.N, self.K = op_a, op_b, M, N, K
        gen = np.random.default_rng(seed)
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

    def reference_bits(self, name):
        """The named configuration on dense op(A), op(B) copies."""
        a = torch.from_numpy(np.ascontiguousarray(self.A.view if self.op_a == "N" else self.A.view.T)).cuda()
        b = torch.from_numpy(np.ascontiguousarray(self.B.view if self.op_b == "N" else self.B.view.T)).cuda()
        out = binding.gemm(a, b, variant=variant_number(name))
        torch.cuda.synchronize()
        return out.cpu().numpy()


def default_name(M, N, K):
    return binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(M, N, K))


def test_scheduled_kernels_are_the_default_for_their_shapes():
    for shape in [(4096, 4096, 32), (4096, 8192, 96), (8192, 8192, 8192), (7940, 8132, 32), (8132, 7940, 64),
                  (4096, 4096, 100), (4096, 4096, 4), (8192, 8192, 8100)]:
        assert default_name(*shape) == KERNELS["tile256"][0], shape
    for shape in [(2048, 2048, 32), (1500, 2044, 64), (2052, 3000, 96), (4100, 6200, 160), (8200, 8200, 64),
                  (2048, 2048, 100), (2052, 3000, 4)]:
        assert default_name(*shape) == KERNELS["tile128"][0], shape
    for shape in [(4096, 4096, 33), (8194, 8192, 64), (8192, 8193, 64)]:
        assert default_name(*shape) == KERNELS["tile256"][1], shape


FULL = {
    # K = 32 (one phase: prologue and the peeled last steps only), K = 64
    # (two phases) and more; full tiles and edge tiles in both dimensions;
    # a last phase past K with one (K = 4), two (36) and four (100) phases
    "tile256": [(4096, 4096, 32), (4096, 4096, 64), (7940, 8132, 32), (4096, 4096, 100), (4096, 4096, 36),
                (7940, 8132, 4)],
    "tile128": [(2048, 2048, 32), (1500, 2044, 64), (2052, 3000, 96), (2048, 2048, 100), (1500, 2044, 36),
                (2052, 3000, 4)],
}


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("kernel", sorted(KERNELS))
def test_scheduled_full_oracle(kernel, ops, dist):
    """Every entry against the oracle product."""
    op_a, op_b = ops
    name, same_tile = KERNELS[kernel]
    for (M, N, K) in FULL[kernel]:
        assert default_name(M, N, K) == name
        prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, len(op_a + op_b), dist == "int", ord(op_a[0])])
        Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
        say(f"sched full oracle {kernel} {op_a}{op_b} {dist} {(M, N, K)}")
        C = prob.run()
        check_padding_untouched(C)
        what = f"sched {kernel} {op_a}{op_b} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, Cref, what)
        else:
            check_close(C.view, Cref, S, what)
        assert np.array_equal(C.view, prob.reference_bits(same_tile)), what + ": bits differ from " + same_tile


SAMPLED = [
    # kernel, shape, offset, (pad A, pad B, pad C): aligned, then dword-offset and padded
    ("tile256", (4096, 8192, 96), 0, (0, 0, 0)),
    ("tile256", (8192, 4096, 544), 1, (3, 5, 7)),
    ("tile256", (4096, 4096, 256), 3, (1, 2, 1)),
    ("tile256", (7940, 8132, 160), 1, (3, 5, 7)),
    ("tile256", (8132, 7940, 96), 0, (0, 0, 0)),
    ("tile128", (4000, 6000, 1024), 0, (0, 0, 0)),
    ("tile128", (5000, 5004, 128), 1, (3, 5, 7)),
    ("tile128", (4100, 6200, 160), 3, (1, 2, 1)),
    ("tile256", (8192, 4096, 2020), 1, (3, 5, 7)),
    ("tile128", (4000, 6000, 1020), 0, (0, 0, 0)),
]


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("case", SAMPLED, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])) + f"_off{c[2]}")
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_scheduled_sampled(ops, case, dist):
    op_a, op_b = ops
    kernel, (M, N, K), offset, pad = case
    name, same_tile = KERNELS[kernel]
    assert default_name(M, N, K) == name
    prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, offset, len(op_a + op_b), dist == "int"],
                   offset, pad)
    ii, jj = inputs.sample_pairs(M, N, 4096, np.random.default_rng([M, N, K, 5]))
    cref, sref = oracle.gemm_entries(prob.A.view, prob.B.view, ii, jj, op_a=op_a, op_b=op_b)
    say(f"sched sampled {kernel} {op_a}{op_b} {dist} {(M, N, K)} offset={offset} pad={pad}")
    C = prob.run()
    check_padding_untouched(C)
    what = f"sched {kernel} {op_a}{op_b} {dist} {(M, N, K)} offset {offset}"
    if dist == "int":
        check_exact(C.view[ii, jj], cref, what)
    else:
        check_close(C.view[ii, jj], cref, sref, what)
    assert np.all(np.isfinite(C.view))
    assert np.array_equal(C.view, prob.reference_bits(same_tile)), what + ": bits differ from " + same_tile
