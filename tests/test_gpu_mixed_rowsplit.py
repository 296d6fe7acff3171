"""The row-split configuration (mixed256x256_rowsplit): the rows of op(A)
that fill all but the last round of 256 CUs with 256 x 256 tiles of the
16 x 16 x 32 scheduled kernel, the remaining rows on k-split 128 x 128
tiles (at most 256 of them), on 160 x 160 tiles (if they need no more
rounds of 256 CUs than 192 x 192 ones) or on 192 x 192 tiles, against the
16-bit oracle: exact on integer inputs, within 1e-5 S on uniform ones.

The shapes put the split at 3840 rows with 512 left (k-split rest), at
3584 with 1024 left (160 x 160 rest), at 3328 with 1280 left and K % 8 = 2
(160 x 160 rest: the k-split kernel takes K a multiple of 8 only), at 2560
with 2048 left of 6400 columns (192 x 192 rest: 374 tiles, against 520 of
160 x 160), and edge tiles on both sides with 766 rows left; offset views with padding and 40 rows of NaN
after every factor; every op pair through gemm_mixed_op, bit-identical to
the plain product on transposed copies; problems it does not take
(misaligned views, odd K) run configuration 10's kernels."""
from __future__ import annotations

import pytest
import torch

from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding
from test_gpu_mixed_wide import run, variant_number

pytestmark = pytest.mark.gpu

SPLIT = "mixed256x256_rowsplit"

SHAPES = [(4352, 4352, 64), (4608, 4608, 72), (4608, 4610, 66), (4608, 6400, 64), (4350, 4354, 136)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(SPLIT)
    for (M, N, K) in SHAPES:
        say(f"rowsplit variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 17], variant=v)
        what = f"{SPLIT} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


@pytest.mark.parametrize("case", ["misaligned", "odd_k"])
def test_fallback_for_problems_it_does_not_take(case):
    v = variant_number(SPLIT)
    say(f"rowsplit fallback {case}")
    if case == "misaligned":
        C, ref, _ = run("bf16", "N", "N", 4352, 4352, 40, "int", [1, 2, 7], offset=1, pad=(3, 5, 2), variant=v)
    else:
        C, ref, _ = run("bf16", "N", "N", 4352, 4352, 41, "int", [1, 2, 8], variant=v)
    check_exact(C.view, ref, f"{SPLIT} fallback {case}")
    check_padding_untouched(C)


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
# shapes gemm_mixed_op splits: 289 tiles of 256 (the last round 33), the
# rest on k-split tiles; 324 (68), the rest on 192 x 192 tiles
OP_SHAPES = [(4352, 4352, 40), (4608, 4608, 48)]


@pytest.mark.parametrize("ops", OPS, ids=["".join(o) for o in OPS])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_against_oracle(ops, fmt):
    op_a, op_b = ops
    for (M, N, K) in OP_SHAPES:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == SPLIT, (M, N, K)
        say(f"rowsplit ops {op_a}{op_b} {fmt} {(M, N, K)}")
        C, ref, _ = run(fmt, op_a, op_b, M, N, K, "int", [M, N, K, 18])
        check_exact(C.view, ref, f"{SPLIT} {op_a}{op_b} {fmt} {(M, N, K)}")
        check_padding_untouched(C)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_op_pairs_bit_identical_on_transposed_copies(fmt):
    M, N, K = 4352, 4352, 1024
    gen = torch.Generator(device="cuda").manual_seed(37)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dt)
    Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dt)
    assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == SPLIT
    ref = binding.gemm16(X, Y)
    for op_a, op_b in OPS:
        A = X.t().contiguous() if op_a == "T" else X
        B = Y.t().contiguous() if op_b == "T" else Y
        say(f"rowsplit same bits {op_a}{op_b} {fmt}")
        out = binding.gemm16(A, B, op_a=op_a, op_b=op_b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{op_a}{op_b} differs from the plain product"


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_full_size_sampled(fmt, dist):
    """Shapes gemm_mixed splits at full size (4352^3: the rest on k-split
    tiles; 4608^3: on 192 x 192 tiles), on sampled entries of both parts
    and the whole of the two rows either side of the split."""
    from test_gpu_mixed_wide import run_sampled
    for (M, N, K), split in [((4352, 4352, 4352), 3840), ((4608, 4608, 4608), 3584)]:
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == SPLIT
        say(f"rowsplit sampled {fmt} {dist} {(M, N, K)}")
        C, got, ref, S = run_sampled(fmt, M, N, K, dist, M + 5, rows=(split - 1, split))
        what = f"{SPLIT} {fmt} {dist} {(M, N, K)} sampled"
        if dist == "int":
            check_exact(got, ref, what)
        else:
            check_close(got, ref, S, what)
        check_padding_untouched(C)
