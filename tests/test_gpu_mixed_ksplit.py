"""The 16-bit k-split kernel (64 x 64 tiles whose four waves each run the
whole tile over every fourth 32-deep phase, v_mfma_f32_16x16x32) against the
16-bit oracle: exact on integer inputs, within 1e-5 S on uniform ones; edge
tiles, ragged K (a multiple of 8: the first phase reaches below k = 0),
1 to 9 phases per wave, offset views with padding, and 40 rows of NaN after
every factor (a copy that read memory past a factor instead of taking zeros
would poison a stored result); every op pair gives the same bits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

KS = "mixed64x64_bk32_w4_ksplit"
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
GUARD_ROWS = 40


def variant_number(name):
    for v in range(binding.gemm_mixed_num_variants()):
        if binding.gemm_mixed_variant_name(v) == name:
            return v
    raise KeyError(name)


def stored(op, rows, cols):
    return (rows, cols) if op == "N" else (cols, rows)


def run(fmt, op_a, op_b, M, N, K, dist, seed, offset=2, pad=(4, 6, 2), variant=None):
    """C = op(A) op(B) with guarded, padded, offset operands; returns the
    padded C and the oracle's (C, S)."""
    gen = np.random.default_rng(seed)
    ar, ac = stored(op_a, M, K)
    br, bc = stored(op_b, K, N)
    Ab = inputs.to16(inputs.random_matrix(gen, ar, ac, dist), fmt)
    Bb = inputs.to16(inputs.random_matrix(gen, br, bc, dist), fmt)
    A = inputs.padded16(Ab, ac + pad[0], offset, fmt, guard=GUARD_ROWS * (ac + pad[0]) + 64)
    B = inputs.padded16(Bb, bc + pad[1], offset, fmt, guard=GUARD_ROWS * (bc + pad[1]) + 64)
    ldc = N + pad[2]
    C0 = inputs.padded_output(M, N, ldc, 1)
    a = torch.from_numpy(A.buf.view(np.int16)).cuda()
    b = torch.from_numpy(B.buf.view(np.int16)).cuda()
    c = torch.from_numpy(C0.buf).cuda()
    args = (fmt, M, N, K, a.data_ptr() + 2 * offset, A.ld, b.data_ptr() + 2 * offset, B.ld, c.data_ptr() + 4, ldc)
    if variant is not None:
        binding.gemm_mixed_variant(variant, *args)
    else:
        binding.gemm_mixed_op(op_a, op_b, *args)
    torch.cuda.synchronize()
    C = inputs.Padded(c.cpu().numpy(), M, N, ldc, 1)
    ref, S = oracle.gemm16(fmt, A.view, B.view, threads=8, op_a=op_a, op_b=op_b)
    return C, ref, S


# (M, N, K): edge tiles on both sides and K % 32 in {0, 8, 16, 24}; phases
# per wave from 1 (K <= 128) to 9
SHAPES = [(64, 64, 8), (64, 64, 32), (70, 130, 40), (128, 66, 136), (130, 200, 264), (250, 190, 520),
          (100, 300, 1000), (200, 66, 1152), (66, 260, 1024)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(KS)
    for (M, N, K) in SHAPES:
        say(f"ksplit16 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 5], variant=v)
        what = f"{KS} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


# shapes gemm_mixed_op gives to the k-split kernel
OP_SHAPES = [(1024, 1024, 4096), (576, 320, 2056), (700, 130, 1032)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    """Every op pair on shapes gemm_mixed_op gives to the k-split kernel:
    exact on integer data, within 1e-5 S on uniform data."""
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == KS, (M, N, K)
        for dist in ("int", "uniform"):
            say(f"ksplit16 ops {op_a}{op_b} {fmt} {dist} {(M, N, K)}")
            C, ref, S = run(fmt, op_a, op_b, M, N, K, dist, [M, N, K, 6, dist == "int"])
            what = f"{KS} {op_a}{op_b} {fmt} {dist} {(M, N, K)}"
            if dist == "int":
                check_exact(C.view, ref, what)
            else:
                check_close(C.view, ref, S, what)
            check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt):
    """For a given M, N, K the summation order does not depend on how the
    factors are stored: gemm_mixed_op on explicitly transposed copies gives
    gemm_mixed's bits."""
    M, N, K = 576, 320, 2056
    gen = torch.Generator(device="cuda").manual_seed(17)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"ksplit16 same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"


def test_misaligned_operands_fall_back_correctly():
    """A 2-byte-aligned view is not for the k-split kernel's 16-byte copies:
    configuration 9 then runs the element-wise 64 x 64 kernel, still exact."""
    v = variant_number(KS)
    say("ksplit16 misaligned fallback")
    C, ref, _ = run("bf16", "N", "N", 130, 200, 264, "int", [1, 2, 3], offset=1, pad=(3, 5, 2), variant=v)
    check_exact(C.view, ref, "misaligned fallback")
    check_padding_untouched(C)
