"""The scheduled 16 x 16 x 32 kernel on 192 x 192 tiles (configuration
mixed192x192_bk64_w4_wide: four waves of 96 x 96) against the 16-bit
oracle: exact on integer inputs, within 1e-5 S on uniform ones.

The shapes cover one tile and one phase, K % 64 in {8, 0, 2, 8, ...} (a last
phase reaching past K; K % 8 != 0 masks the last chunk of a k-contiguous
factor), edge tiles on both sides with every residue of a 96-wide wave span,
up to 6 x 4 tiles and 16 phases, offset views with padding, and 40 rows of
NaN after every factor (a copy that read memory past a factor instead of
taking zeros, or an mn-contiguous copy's lanes beyond the tile, would poison
a stored result); a second call gives the same bits; problems the kernel
does not take (misaligned views, odd K) run the 256 x 256 fallbacks."""
from __future__ import annotations

import pytest
import torch

from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding
from test_gpu_mixed_wide import run, variant_number

pytestmark = pytest.mark.gpu

W192 = "mixed192x192_bk64_w4_wide"

# (M, N, K): one tile, one phase; one tile, one whole phase; 2 x 3 tiles,
# K % 64 = 8; edge tiles whose last wave span is partly or wholly empty
# (M % 192 = 16, N % 192 = 6), K % 8 = 2; 5 x 2 tiles; 4 x 6 tiles with 16
# phases; a last phase of 6 k
SHAPES = [(192, 192, 8), (192, 192, 64), (300, 520, 136), (400, 390, 130), (770, 258, 200),
          (600, 1030, 1000), (1000, 600, 518)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(W192)
    for (M, N, K) in SHAPES:
        say(f"wide192 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 14], variant=v)
        what = f"{W192} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


def test_variant_repeats_bit_for_bit():
    """Fixed k order: a second call gives the same bits."""
    v = variant_number(W192)
    gen = torch.Generator(device="cuda").manual_seed(8)
    X = (torch.rand((770, 1000), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    Y = (torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    say("wide192 repeat")
    first = binding.gemm16(X, Y, variant=v)
    second = binding.gemm16(X, Y, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


@pytest.mark.parametrize("case", ["misaligned", "odd_k"])
def test_fallback_for_problems_it_does_not_take(case):
    """A 2-byte-aligned view, or an odd K: the configuration runs the
    8-wave 256 x 256 kernels, still exact."""
    v = variant_number(W192)
    say(f"wide192 fallback {case}")
    if case == "misaligned":
        C, ref, _ = run("bf16", "N", "N", 300, 520, 136, "int", [1, 2, 5], offset=1, pad=(3, 5, 2), variant=v)
    else:
        C, ref, _ = run("bf16", "N", "N", 300, 520, 137, "int", [1, 2, 6], variant=v)
    check_exact(C.view, ref, f"{W192} fallback {case}")
    check_padding_untouched(C)


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# shapes gemm_mixed_op gives to this kernel: 225 tiles of 192 (fewer than
# 128 of 256, more than 256 of 128 or of 160); 15 x 16 edge tiles with K %
# 8 = 2
OP_SHAPES = [(2816, 2816, 64), (2700, 2900, 130)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    """Every op pair through gemm_mixed_op, which gives these shapes to this
    kernel: exact on integer data, within 1e-5 S on uniform data."""
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W192, (M, N, K)
        for dist in ("int", "uniform"):
            say(f"wide192 ops {op_a}{op_b} {fmt} {dist} {(M, N, K)}")
            C, ref, S = run(fmt, op_a, op_b, M, N, K, dist, [M, N, K, 15, dist == "int"])
            what = f"{W192} {op_a}{op_b} {fmt} {dist} {(M, N, K)}"
            if dist == "int":
                check_exact(C.view, ref, what)
            else:
                check_close(C.view, ref, S, what)
            check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt):
    """The k order does not depend on how a factor is stored: gemm_mixed_op
    on explicitly transposed copies gives the bits of the plain product."""
    M, N, K = 3072, 3072, 1024
    gen = torch.Generator(device="cuda").manual_seed(31)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W192
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"wide192 same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_full_size_sampled(fmt, dist):
    """Shapes gemm_mixed gives to this kernel at full size (3072^3: 256
    tiles; 4100^2 x 4096: edge tiles, two rounds), on sampled entries."""
    from test_gpu_mixed_wide import run_sampled
    for (M, N, K) in [(3072, 3072, 3072), (4100, 4100, 4096)]:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W192
        say(f"wide192 sampled {fmt} {dist} {(M, N, K)}")
        C, got, ref, S = run_sampled(fmt, M, N, K, dist, M + 3)
        what = f"{W192} {fmt} {dist} {(M, N, K)} sampled"
        if dist == "int":
            check_exact(got, ref, what)
        else:
            check_close(got, ref, S, what)
        check_padding_untouched(C)
