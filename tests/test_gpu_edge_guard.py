"""The scheduled kernels' zero copies never depend on memory past a factor.

Where a copy of the four-wave fp32 kernels (256 x 256, 128 x 128 and 64 x 64 tiles),
the k-split fp32 kernel or the scheduled 16-bit kernel must bring zeros -- a
last phase that reaches past K, phase 0 of the k-split kernel reaching below
k = 0, the column overhang of an edge tile -- its per-lane offset lies past
the end of the factor's buffer descriptor by itself.  Here every stored
factor is followed by a guard of NaN at least 32 rows long (more than any
phase can reach past the end) and preceded by NaN words: a copy that read
memory there instead of taking zeros would put NaN into a stored result.
Integer inputs make the result exact; every op pair runs each kernel on a
shape with ragged K (not a multiple of the phase depth) and edge tiles on
both sides.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
GUARD_ROWS = 40
# kernel -> (M, N, K): shapes gemm_f32 / gemm_mixed give to that kernel,
# K not a multiple of the kernel's phase depth (32 fp32, 64 16-bit), M and N
# not multiples of the tile.
FP32_CASES = {
    "mfma256x256_bk32_w2x2_sched": (4092, 4092, 100),
    "mfma128x128_bk32_w2x2_sched": (1532, 1404, 164),
    "mfma64x64_bk32_w1x1_k4_sched": (556, 572, 1004),
    "mfma64x64_bk32_w2x2_sched": (1532, 1028, 388),
}
MIXED_CASES = {"mixed256x256_bk64_w4_wide": (3580, 3330, 200), "mixed192x192_bk64_w4_wide": (3068, 3068, 200),
               "mixed160x160_bk64_w4_wide": (2390, 2470, 200)}


def stored(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


def guarded(dense, ld, offset, fill):
    return inputs.padded(dense, ld, offset, fill=fill, guard=GUARD_ROWS * ld + 64)


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("kernel", sorted(FP32_CASES))
def test_fp32_zero_copies_read_no_guard(kernel, ops):
    M, N, K = FP32_CASES[kernel]
    assert binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(M, N, K)) == kernel
    op_a, op_b = ops
    gen = np.random.default_rng([M, N, K, len(kernel)])
    ar, ac = stored(op_a, M, K)
    br, bc = stored(op_b, K, N)
    A = guarded(inputs.random_matrix(gen, ar, ac, "int"), ac + 3, 1, np.nan)
    B = guarded(inputs.random_matrix(gen, br, bc, "int"), bc + 5, 1, np.nan)
    ref, _ = oracle.gemm(A.view, B.view, threads=8, op_a=op_a, op_b=op_b)
    C0 = inputs.padded_output(M, N, N + 2, 1)
    a, b, c = (torch.from_numpy(x.buf).cuda() for x in (A, B, C0))
    say(f"edge guard fp32 kernel={kernel} ops={op_a}{op_b} M={M} N={N} K={K}")
    binding.gemm_f32_op(op_a, op_b, M, N, K, a.data_ptr() + 4, A.ld, b.data_ptr() + 4, B.ld,
                        c.data_ptr() + 4, N + 2)
    torch.cuda.synchronize()
    C = inputs.Padded(c.cpu().numpy(), M, N, N + 2, 1)
    check_exact(C.view, ref, f"{kernel} {op_a}{op_b}")
    check_padding_untouched(C)


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", sorted(MIXED_CASES))
def test_mixed_zero_copies_read_no_guard(kernel, fmt, ops):
    M, N, K = MIXED_CASES[kernel]
    assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == kernel
    op_a, op_b = ops
    gen = np.random.default_rng([M, N, K, 16])
    ar, ac = stored(op_a, M, K)
    br, bc = stored(op_b, K, N)
    Ab = inputs.to16(inputs.random_matrix(gen, ar, ac, "int"), fmt)
    Bb = inputs.to16(inputs.random_matrix(gen, br, bc, "int"), fmt)
    # even leading dimensions and an offset of two elements keep the
    # scheduled kernels' 4-byte alignment
    A = inputs.padded16(Ab, ac + 4, 2, fmt, guard=GUARD_ROWS * (ac + 4) + 64)
    B = inputs.padded16(Bb, bc + 6, 2, fmt, guard=GUARD_ROWS * (bc + 6) + 64)
    ref, _ = oracle.gemm16(fmt, A.view, B.view, threads=8, op_a=op_a, op_b=op_b)
    C0 = inputs.padded_output(M, N, N + 2, 1)
    a = torch.from_numpy(A.buf.view(np.int16)).cuda()
    b = torch.from_numpy(B.buf.view(np.int16)).cuda()
    c = torch.from_numpy(C0.buf).cuda()
    say(f"edge guard mixed kernel={kernel} fmt={fmt} ops={op_a}{op_b} M={M} N={N} K={K}")
    binding.gemm_mixed_op(op_a, op_b, fmt, M, N, K, a.data_ptr() + 4, A.ld, b.data_ptr() + 4, B.ld,
                          c.data_ptr() + 4, N + 2)
    torch.cuda.synchronize()
    C = inputs.Padded(c.cpu().numpy(), M, N, N + 2, 1)
    check_exact(C.view, ref, f"{kernel} {fmt} {op_a}{op_b}")
    check_padding_untouched(C)
