"""The scheduled 256 x 256 kernel on v_mfma_f32_16x16x32 (configuration
mixed256x256_bk64_w4_wide) against the 16-bit oracle: exact on integer
inputs, within 1e-5 S on uniform ones; edge tiles on both sides, K % 64 in
{0, 8, 40, ...} (a last phase reaching past K) and K % 8 != 0 (the last
chunk of a k-contiguous factor masked), one to sixteen phases,
offset views with padding, and 40 rows of NaN after every factor (a copy
that read memory past a factor instead of taking zeros would poison a stored
result); every op pair through gemm_mixed_op, with the bits of the plain
product on explicitly transposed copies; a second call gives the same
bits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

WIDE = "mixed256x256_bk64_w4_wide"
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


# (M, N, K): one tile and one phase up to 4 x 3 tiles and 16 phases; edge
# tiles on both sides; K % 64 in {8, 0, 8, 0, 8, 40, 8}
SHAPES = [(256, 256, 8), (256, 256, 64), (300, 520, 136), (512, 512, 128), (770, 258, 200),
          (520, 1030, 1000), (1024, 768, 520)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(WIDE)
    for (M, N, K) in SHAPES:
        say(f"wide16 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 9], variant=v)
        what = f"{WIDE} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


# K not a multiple of 8: the chunk of A (k-contiguous) that holds k = K - 1
# also holds values past K, which the last phase masks; (M, N, K, pad of A's
# leading dimension): K % 64 in {4, 10, 44, 46}, the straddling chunk in step
# 0 or step 1 of the last phase; then odd K with an even leading dimension,
# which the configuration hands to its fallback (the last row's last value
# would share a dword with the bytes past the descriptor's end)
RAGGED = [(256, 256, 4, 4), (300, 520, 138, 4), (520, 1030, 1004, 4), (770, 258, 46, 6), (1024, 768, 517, 5),
          (258, 516, 63, 3)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_ragged_k(fmt, dist):
    v = variant_number(WIDE)
    for (M, N, K, pa) in RAGGED:
        say(f"wide16 ragged K {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 7], pad=(pa, 6, 2), variant=v)
        what = f"{WIDE} ragged {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


def test_variant_repeats_bit_for_bit():
    """Fixed k order: a second call gives the same bits."""
    v = variant_number(WIDE)
    gen = torch.Generator(device="cuda").manual_seed(5)
    X = (torch.rand((770, 1000), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    Y = (torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    say("wide16 repeat")
    first = binding.gemm16(X, Y, variant=v)
    second = binding.gemm16(X, Y, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# shapes gemm_mixed_op gives to the kernel (at least 128 tiles of 256 x 256,
# one round of them against two of 192 x 192); edge tiles in N, then in
# both; the last two with K % 8 != 0 (a k-contiguous factor's last chunk
# straddles K in step 0, then step 1, of the last phase)
OP_SHAPES = [(3584, 3330, 72), (3580, 3336, 136), (3580, 3336, 76), (3584, 3330, 110)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    """Every op pair through gemm_mixed_op, which gives these shapes to this
    kernel: exact on integer data, within 1e-5 S on uniform data."""
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == WIDE, (M, N, K)
        for dist in ("int", "uniform"):
            say(f"wide16 ops {op_a}{op_b} {fmt} {dist} {(M, N, K)}")
            C, ref, S = run(fmt, op_a, op_b, M, N, K, dist, [M, N, K, 8, dist == "int"])
            what = f"{WIDE} {op_a}{op_b} {fmt} {dist} {(M, N, K)}"
            if dist == "int":
                check_exact(C.view, ref, what)
            else:
                check_close(C.view, ref, S, what)
            check_padding_untouched(C)


@pytest.mark.parametrize("K", [1000, 1002])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt, K):
    """The k order inside each instruction does not depend on how a factor
    is stored: gemm_mixed_op on explicitly transposed copies gives the bits
    of the plain product (also with K % 8 != 0, where a k-contiguous
    factor's last chunk is masked)."""
    M, N = 3072, 2816
    gen = torch.Generator(device="cuda").manual_seed(23)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"wide16 same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"


def test_misaligned_operands_fall_back_correctly():
    """A 2-byte-aligned view is not for the kernel's 16-byte copies: the
    configuration then runs the element-wise 8-wave kernel, still exact."""
    v = variant_number(WIDE)
    say("wide16 misaligned fallback")
    C, ref, _ = run("bf16", "N", "N", 300, 520, 136, "int", [1, 2, 3], offset=1, pad=(3, 5, 2), variant=v)
    check_exact(C.view, ref, "misaligned fallback")
    check_padding_untouched(C)


def run_sampled(fmt, M, N, K, dist, seed, count=4096, rows=(), variant=None):
    """gemm_mixed (or configuration `variant`) on padded, offset, guarded
    operands of a full-size shape,
    checked on `count` sampled entries plus the corners, every tile edge's
    last row and column and the whole of each row in `rows`: returns (C,
    the results at those entries, the oracle's values, the oracle's S)."""
    gen = np.random.default_rng(seed)
    Ab = inputs.to16(inputs.random_matrix(gen, M, K, dist), fmt)
    Bb = inputs.to16(inputs.random_matrix(gen, K, N, dist), fmt)
    A = inputs.padded16(Ab, K + 4, 2, fmt, guard=GUARD_ROWS * (K + 4) + 64)
    B = inputs.padded16(Bb, N + 6, 2, fmt, guard=GUARD_ROWS * (N + 6) + 64)
    ldc = N + 2
    C0 = inputs.padded_output(M, N, ldc, 1)
    a = torch.from_numpy(A.buf.view(np.int16)).cuda()
    b = torch.from_numpy(B.buf.view(np.int16)).cuda()
    c = torch.from_numpy(C0.buf).cuda()
    args = (fmt, M, N, K, a.data_ptr() + 4, A.ld, b.data_ptr() + 4, B.ld, c.data_ptr() + 4, ldc)
    if variant is not None:
        binding.gemm_mixed_variant(variant, *args)
    else:
        binding.gemm_mixed(*args)
    torch.cuda.synchronize()
    C = inputs.Padded(c.cpu().numpy(), M, N, ldc, 1)
    ii, jj = inputs.sample_pairs(M, N, count, np.random.default_rng([seed, 1]), tiles=(64, 128, 160, 192, 256))
    if len(rows):
        ii = np.concatenate([ii, np.repeat(np.asarray(rows, np.int64), N)])
        jj = np.concatenate([jj, np.tile(np.arange(N, dtype=np.int64), len(rows))])
    ref, S = oracle.gemm16_entries(fmt, A.view, B.view, ii, jj)
    return C, C.view[ii, jj], ref, S
