"""128 x 128 tiles whose four waves each run the whole tile over every fourth
32-deep phase (configuration mixed128x128_bk32_w4_ksplit) against the
16-bit oracle: exact on integer inputs, within 1e-5 S on uniform ones.

The shapes cover one phase in all (three waves without a phase), K % 32 != 0
(phase 0 reaching below k = 0), one phase per wave (an odd count: a position
that copies zeros), two, three and seventeen phases for a wave, edge tiles
on both sides, offset views with padding, and 40 rows of NaN after every
factor (a copy that read memory past a factor instead of taking zeros would
poison a stored result); a second call gives the same bits; problems the
kernel does not take (misaligned views, K not a multiple of 8) run the
128 x 128 fallback."""
from __future__ import annotations

import pytest
import torch

from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding
from test_gpu_mixed_wide import run, variant_number

pytestmark = pytest.mark.gpu

KS128 = "mixed128x128_bk32_w4_ksplit"

# (M, N, K): phases of 32 k over four waves -- K = 8: one phase in all;
# 40: two, the first reaching below k = 0; 128: one per wave; 160: wave 0
# two, the others one; 288: wave 0 three; 1000: eight each; 2056: wave 0
# seventeen
SHAPES = [(128, 128, 8), (128, 128, 40), (300, 520, 128), (256, 384, 160), (520, 1030, 288), (1000, 1000, 1000),
          (384, 256, 2056)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(KS128)
    for (M, N, K) in SHAPES:
        say(f"ksplit128 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 12], variant=v)
        what = f"{KS128} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


def test_variant_repeats_bit_for_bit():
    """Fixed k order: a second call gives the same bits."""
    v = variant_number(KS128)
    gen = torch.Generator(device="cuda").manual_seed(6)
    X = (torch.rand((770, 1000), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    Y = (torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    say("ksplit128 repeat")
    first = binding.gemm16(X, Y, variant=v)
    second = binding.gemm16(X, Y, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


@pytest.mark.parametrize("case", ["misaligned", "k_not_multiple_of_8"])
def test_fallback_for_problems_it_does_not_take(case):
    """A 2-byte-aligned view, or K not a multiple of 8: the configuration
    runs the 128 x 128 fallback, still exact."""
    v = variant_number(KS128)
    say(f"ksplit128 fallback {case}")
    if case == "misaligned":
        C, ref, _ = run("bf16", "N", "N", 300, 520, 136, "int", [1, 2, 3], offset=1, pad=(3, 5, 2), variant=v)
    else:
        C, ref, _ = run("bf16", "N", "N", 300, 520, 138, "int", [1, 2, 4], variant=v)
    check_exact(C.view, ref, f"{KS128} fallback {case}")
    check_padding_untouched(C)


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# shapes gemm_mixed_op gives to this kernel (128 .. 256 tiles of 128 x 128,
# K >= 1024): 144 tiles; 9 x 17 edge tiles with K % 32 = 8 (wave 0 with
# nine phases, an odd count)
OP_SHAPES = [(1536, 1536, 1024), (1100, 2100, 1032)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    """Every op pair through gemm_mixed_op, which gives these shapes to this
    kernel: exact on integer data, within 1e-5 S on uniform data."""
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == KS128, (M, N, K)
        for dist in ("int", "uniform"):
            say(f"ksplit128 ops {op_a}{op_b} {fmt} {dist} {(M, N, K)}")
            C, ref, S = run(fmt, op_a, op_b, M, N, K, dist, [M, N, K, 13, dist == "int"])
            what = f"{KS128} {op_a}{op_b} {fmt} {dist} {(M, N, K)}"
            if dist == "int":
                check_exact(C.view, ref, what)
            else:
                check_close(C.view, ref, S, what)
            check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt):
    """The k order does not depend on how a factor is stored: gemm_mixed_op
    on explicitly transposed copies gives the bits of the plain product."""
    M, N, K = 2048, 2048, 1024
    gen = torch.Generator(device="cuda").manual_seed(29)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == KS128
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"ksplit128 same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"
