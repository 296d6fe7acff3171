"""The 64 x 64 kernel whose four waves split the phases of one tile (each
wave the whole tile over every fourth 32-deep phase, partial tiles added in
wave order), which gemm_f32 and gemm_f32_op run for K, M and N multiples of 4
where its cost model wins (K >= 448) or in place of the split-phase tiles
(K >= 384).  Its phases are aligned to the end of K, so with K not a multiple
of 32 the first phase reaches below k = 0 and those lanes copy zeros.

Checked against the oracle (every entry on small problems, sampled entries on
large ones; exact on integer inputs) for all four op pairs, on aligned and on
padded, dword-offset operands whose pad words are NaN; bit for bit across the
op pairs (explicitly transposed copies) and across repeated calls; through the
diagnostic variant (op N only) for K from 4 to 388, where some waves have no
phase or one or two; and with an infinity planted at k = K - 1, which must
reach only its own row or column of C."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

KS = "mfma64x64_bk32_w1x1_k4_sched"
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def variant_number(name):
    for d in range(binding.gemm_f32_num_diagnostic_variants()):
        if binding.gemm_f32_variant_name(binding.DIAGNOSTIC_BASE + d) == name:
            return binding.DIAGNOSTIC_BASE + d
    raise KeyError(name)


def default_name(M, N, K):
    return binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(M, N, K))


def stored_shape(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


class Problem:
    """op(A) x op(B) on padded device buffers (pad words NaN, C sentinels)."""

    def __init__(self, op_a, op_b, M, N, K, dist, seed, offset=0, pad=(0, 0, 0), dense=None):
        self.op_a, self.op_b, self.M, self.N, self.K = op_a, op_b, M, N, K
        gen = np.random.default_rng(seed)
        ar, ac = stored_shape(op_a, M, K)
        br, bc = stored_shape(op_b, K, N)
        a, b = dense if dense is not None else (inputs.random_matrix(gen, ar, ac, dist),
                                                inputs.random_matrix(gen, br, bc, dist))
        self.A = inputs.padded(a, ac + pad[0], offset)
        self.B = inputs.padded(b, bc + pad[1], offset)
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

    def plain_bits(self):
        """gemm_f32 (op N, N) on dense copies of op(A) and op(B)."""
        a = torch.from_numpy(np.ascontiguousarray(self.A.view if self.op_a == "N" else self.A.view.T)).cuda()
        b = torch.from_numpy(np.ascontiguousarray(self.B.view if self.op_b == "N" else self.B.view.T)).cuda()
        out = binding.gemm(a, b)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def test_kernel_is_the_default_for_its_shapes():
    for shape in [(1000, 1000, 1000), (560, 548, 1000), (540, 516, 516), (5120, 5120, 5120),
                  (2300, 2300, 2304), (1000, 2000, 1000), (4100, 4104, 4100), (2000, 1000, 996)]:
        assert default_name(*shape) == KS, shape
    for shape in [(1000, 1000, 380), (1002, 1000, 1000), (1000, 1000, 1001), (8192, 8192, 8192),
                  (2048, 2048, 2048)]:
        assert default_name(*shape) != KS, shape


FULL = [
    # 9 x 9 tiles with ragged edges and K % 32 = 8 (first phase partial),
    # 9 x 9 tiles with K % 32 = 4, 16 x 16 tiles with K a multiple of 32
    # (more than 1024 output tiles of 16 x 16 each, so not the small-tile
    # kernels)
    (560, 548, 1000),
    (540, 516, 516),
    (1000, 1000, 512),
]


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("shape", FULL, ids=lambda s: "x".join(map(str, s)))
def test_full_oracle(shape, ops, dist):
    """Every entry against the oracle product; the same bits on a second call
    and as the op N, N product of transposed copies."""
    op_a, op_b = ops
    M, N, K = shape
    assert default_name(M, N, K) == KS
    prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, len(op_a + op_b), dist == "int", ord(op_a), 7])
    Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
    say(f"ksplit full {op_a}{op_b} {dist} {shape}")
    C = prob.run()
    check_padding_untouched(C)
    what = f"ksplit {op_a}{op_b} {dist} {shape}"
    if dist == "int":
        check_exact(C.view, Cref, what)
    else:
        check_close(C.view, Cref, S, what)
    again = prob.run()
    assert np.array_equal(C.view, again.view), what + ": a second call gave other bits"
    assert np.array_equal(C.view, prob.plain_bits()), what + ": bits differ from the op N, N product"


SAMPLED = [
    # shape, offset, (pad A, pad B, pad C)
    ((1000, 1000, 1000), 1, (3, 5, 7)),
    ((5120, 5120, 5120), 0, (0, 0, 0)),
    ((4100, 4104, 4100), 3, (1, 2, 1)),
    ((2000, 1000, 996), 1, (4, 0, 3)),
]


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("case", SAMPLED, ids=lambda c: "x".join(map(str, c[0])) + f"_off{c[1]}")
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_sampled(ops, case, dist):
    op_a, op_b = ops
    (M, N, K), offset, pad = case
    assert default_name(M, N, K) == KS
    prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, offset, len(op_a + op_b), dist == "int", 7],
                   offset, pad)
    ii, jj = inputs.sample_pairs(M, N, 4096, np.random.default_rng([M, N, K, 11]))
    cref, sref = oracle.gemm_entries(prob.A.view, prob.B.view, ii, jj, op_a=op_a, op_b=op_b)
    say(f"ksplit sampled {op_a}{op_b} {dist} {(M, N, K)} offset={offset} pad={pad}")
    C = prob.run()
    check_padding_untouched(C)
    what = f"ksplit {op_a}{op_b} {dist} {(M, N, K)} offset {offset}"
    if dist == "int":
        check_exact(C.view[ii, jj], cref, what)
    else:
        check_close(C.view[ii, jj], cref, sref, what)
    assert np.all(np.isfinite(C.view)), what


# K = 4 .. 388: waves with no phase (K <= 96), one, two, three; K % 32 in
# {0, 4, 8, 28}.
SMALL_K = [4, 8, 28, 32, 36, 64, 96, 100, 128, 132, 260, 388]


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("K", SMALL_K)
def test_variant_short_k(K, dist):
    """Through the diagnostic variant (op N, N): 3 x 4 tiles with ragged
    edges, padded and offset operands."""
    M, N = 136, 200
    gen = np.random.default_rng([M, N, K, dist == "int", 13])
    A = inputs.padded(inputs.random_matrix(gen, M, K, dist), K + 3, 1)
    B = inputs.padded(inputs.random_matrix(gen, K, N, dist), N + 5, 1)
    Cref, S = oracle.gemm(A.view, B.view, threads=8)
    say(f"ksplit variant {dist} {(M, N, K)}")
    A_dev = torch.from_numpy(A.buf).cuda()
    B_dev = torch.from_numpy(B.buf).cuda()
    C_init = inputs.padded_output(M, N, N + 7, 1)
    C_dev = torch.from_numpy(C_init.buf).cuda()
    binding.gemm_f32_variant(variant_number(KS), M, N, K, A_dev.data_ptr() + 4, A.ld, B_dev.data_ptr() + 4, B.ld,
                             C_dev.data_ptr() + 4, N + 7)
    torch.cuda.synchronize()
    C = inputs.Padded(C_dev.cpu().numpy(), M, N, N + 7, 1)
    check_padding_untouched(C)
    what = f"ksplit variant {dist} {(M, N, K)}"
    if dist == "int":
        check_exact(C.view, Cref, what)
    else:
        check_close(C.view, Cref, S, what)


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("factor", ["A", "B"])
def test_planted_infinity_stays_in_its_row_or_column(ops, factor):
    """op(A)[r, K - 1] = inf makes row r of C non-finite and no other (op(B)
    [K - 1, c]: column c).  A lane of the first, partial phase that read the
    stored row before its own, instead of a zero, would carry the infinity to
    row r + 1 (column c + 1)."""
    op_a, op_b = ops
    M, N, K = 580, 520, 1000                                # K % 32 = 8
    assert default_name(M, N, K) == KS
    gen = np.random.default_rng([M, N, K, len(op_a + op_b), ord(factor)])
    a = inputs.random_matrix(gen, *stored_shape(op_a, M, K), "uniform")
    b = inputs.random_matrix(gen, *stored_shape(op_b, K, N), "uniform")
    r, c = 67, 131
    if factor == "A":
        a[(r, K - 1) if op_a == "N" else (K - 1, r)] = np.inf
    else:
        b[(K - 1, c) if op_b == "N" else (c, K - 1)] = np.inf
    prob = Problem(op_a, op_b, M, N, K, "uniform", None, dense=(a, b))
    say(f"ksplit planted inf in {factor} {op_a}{op_b}")
    C = prob.run().view
    bad = ~np.isfinite(C)
    want = np.zeros_like(bad)
    if factor == "A":
        want[r, :] = True
    else:
        want[:, c] = True
    assert np.array_equal(bad, want), f"non-finite entries outside row/column: {np.argwhere(bad & ~want)[:4]}"
    Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
    check_close(C[~want], Cref[~want], S[~want], f"planted {factor} {op_a}{op_b}")


@pytest.mark.parametrize("shape", [(1000, 1000, 1000), (200, 136, 388), (64, 64, 4)])
def test_timeline_helper_runs_the_same_kernel(shape):
    """The measurement helper's instantiation gives gemm_f32's bits, and every
    wave's five stamps come in order, with its phase count and block."""
    M, N, K = shape
    assert default_name(M, N, K) == KS or shape != (1000, 1000, 1000)
    gen = torch.Generator(device="cuda").manual_seed(11)
    A = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
    B = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
    ref = torch.empty((M, N), device="cuda")
    out = torch.empty((M, N), device="cuda")
    binding.gemm_f32_variant(variant_number(KS), M, N, K, A, K, B, N, ref, N)
    blocks = ((M + 63) // 64) * ((N + 63) // 64)
    tl = torch.zeros(32 * blocks, dtype=torch.int32, device="cuda")
    say(f"ksplit timeline {shape}")
    binding.gemm_f32_ksplit_timeline(M, N, K, A, K, B, N, out, N, tl, tl.numel())
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    rows = tl.view(-1, 8).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    nph = (K + 31) // 32
    for i, r in enumerate(rows):
        steps = [(r[t + 1] - r[t]) & 0xFFFFFFFF for t in range(4)]
        assert all(0 <= d < 100_000_000 for d in steps), (i, r)          # under a second each
        assert r[6] == (max(nph - 1 - i % 4, -1) // 4 + 1 if nph > i % 4 else 0), (i, r)
        assert r[7] == i // 4
