"""The scheduled 16 x 16 x 32 kernel on 160 x 160 tiles (configuration
mixed160x160_bk64_w4_wide: four waves of 80 x 80) against the 16-bit
oracle: exact on integer inputs, within 1e-5 S on uniform ones.

The shapes cover one tile and one phase, K % 64 in {8, 0, 8, 2, 8, ...} (a
last phase reaching past K; K % 8 != 0 masks the last chunk of a
k-contiguous factor), edge tiles whose last 80-wide wave span is empty,
partly filled or whole on either side, up to 7 x 4 tiles and 16 phases,
offset views with padding, and 40 rows of NaN after every factor (a copy
that read memory past a factor instead of taking zeros, or an mn-contiguous
copy's lanes beyond the tile -- 96 of every 256 values -- would poison a
stored result); a second call gives the same bits; problems the kernel does
not take (misaligned views, odd K) run the 256 x 256 fallbacks."""
from __future__ import annotations

import pytest
import torch

from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding
from test_gpu_mixed_wide import run, run_sampled, variant_number

pytestmark = pytest.mark.gpu

W160 = "mixed160x160_bk64_w4_wide"

# (M, N, K): one tile, one phase; one tile, one whole phase; 2 x 4 tiles,
# K % 64 = 8; M % 160 = 80 (the last tile's second wave span empty) and
# N % 160 = 70, K % 8 = 2; M % 160 = 130, N % 160 = 98 (second spans partly
# filled); 4 x 7 tiles with 16 phases; a last phase of 6 k
SHAPES = [(160, 160, 8), (160, 160, 64), (300, 520, 136), (400, 390, 130), (770, 258, 200),
          (600, 1030, 1000), (1000, 600, 518)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(W160)
    for (M, N, K) in SHAPES:
        say(f"wide160 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 16], variant=v)
        what = f"{W160} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


def test_variant_repeats_bit_for_bit():
    """Fixed k order: a second call gives the same bits."""
    v = variant_number(W160)
    gen = torch.Generator(device="cuda").manual_seed(9)
    X = (torch.rand((770, 1000), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    Y = (torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    say("wide160 repeat")
    first = binding.gemm16(X, Y, variant=v)
    second = binding.gemm16(X, Y, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


@pytest.mark.parametrize("case", ["misaligned", "odd_k"])
def test_fallback_for_problems_it_does_not_take(case):
    """A 2-byte-aligned view, or an odd K: the configuration runs the
    8-wave 256 x 256 kernels, still exact."""
    v = variant_number(W160)
    say(f"wide160 fallback {case}")
    if case == "misaligned":
        C, ref, _ = run("bf16", "N", "N", 300, 520, 136, "int", [1, 2, 7], offset=1, pad=(3, 5, 2), variant=v)
    else:
        C, ref, _ = run("bf16", "N", "N", 300, 520, 137, "int", [1, 2, 8], variant=v)
    check_exact(C.view, ref, f"{W160} fallback {case}")
    check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_full_size_sampled(fmt, dist):
    """Full-size shapes on this configuration (2560^3: 256 tiles, one per CU;
    2500 x 2600 x 2046: edge tiles and a last phase of 62 k), on sampled
    entries plus every tile edge."""
    v = variant_number(W160)
    for (M, N, K) in [(2560, 2560, 2560), (2500, 2600, 2046)]:
        say(f"wide160 sampled {fmt} {dist} {(M, N, K)}")
        C, got, ref, S = run_sampled(fmt, M, N, K, dist, M + 5, variant=v)
        what = f"{W160} {fmt} {dist} {(M, N, K)} sampled"
        if dist == "int":
            check_exact(got, ref, what)
        else:
            check_close(got, ref, S, what)
        check_padding_untouched(C)


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# shapes gemm_mixed_op gives to this kernel: 225 tiles of 160 (144 of 192,
# one round either way); 14 x 16 edge tiles (M % 160 = 120, N % 160 = 100)
# with K % 8 = 2
OP_SHAPES = [(2304, 2304, 64), (2200, 2500, 130)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    """Every op pair through gemm_mixed_op, which gives these shapes to this
    kernel: exact on integer data, within 1e-5 S on uniform data."""
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W160, (M, N, K)
        for dist in ("int", "uniform"):
            say(f"wide160 ops {op_a}{op_b} {fmt} {dist} {(M, N, K)}")
            C, ref, S = run(fmt, op_a, op_b, M, N, K, dist, [M, N, K, 17, dist == "int"])
            what = f"{W160} {op_a}{op_b} {fmt} {dist} {(M, N, K)}"
            if dist == "int":
                check_exact(C.view, ref, what)
            else:
                check_close(C.view, ref, S, what)
            check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt):
    """The k order does not depend on how a factor is stored: gemm_mixed_op
    on explicitly transposed copies gives the bits of the plain product."""
    M, N, K = 2560, 2560, 1024
    gen = torch.Generator(device="cuda").manual_seed(33)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W160
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"wide160 same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"


@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_default_pick_full_size_sampled(dist):
    """gemm_mixed's own choice at 1280 x 5120 x 2048 (256 tiles of 160) and
    at a ragged K (1000 x 2000 x 500, K % 8 = 4), on sampled entries."""
    for (M, N, K) in [(1280, 5120, 2048), (1000, 2000, 500)]:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == W160
        say(f"wide160 default sampled {dist} {(M, N, K)}")
        C, got, ref, S = run_sampled("bf16", M, N, K, dist, M + 7)
        what = f"{W160} default {dist} {(M, N, K)} sampled"
        if dist == "int":
            check_exact(got, ref, what)
        else:
            check_close(got, ref, S, what)
        check_padding_untouched(C)
