"""The four-stage form of the 16 x 16 x 32 scheduled kernel (configuration
mixed256x256_bk32_w4_wide4stage: 32-deep phases in four LDS stages, the last
32-k block first, zero phases up to a multiple of four) against the 16-bit
oracle: exact on integer inputs, within 1e-5 S on uniform ones; edge tiles,
K % 32 in {0, 8, 24}, 1 to 32 blocks (0 to 3 zero phases), offset views with
padding and 40 rows of NaN after every factor; a second call gives the same
bits; misaligned operands run the element-wise 8-wave kernel."""
from __future__ import annotations

import pytest
import torch

from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding
from test_gpu_mixed_wide import run, variant_number

pytestmark = pytest.mark.gpu

WIDE4 = "mixed256x256_bk32_w4_wide4stage"
# (M, N, K): blocks of 32 k: 1, 1, 5, 4, 7, 32, 17 (zero phases 3, 3, 3, 0, 1, 0, 3)
SHAPES = [(256, 256, 8), (256, 256, 24), (300, 520, 136), (512, 512, 128), (770, 258, 200),
          (520, 1030, 1000), (1024, 768, 520)]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(fmt, dist):
    v = variant_number(WIDE4)
    for (M, N, K) in SHAPES:
        say(f"wide4 variant {fmt} {dist} {(M, N, K)}")
        C, ref, S = run(fmt, "N", "N", M, N, K, dist, [M, N, K, 10], variant=v)
        what = f"{WIDE4} {fmt} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, ref, what)
        else:
            check_close(C.view, ref, S, what)
        check_padding_untouched(C)


def test_variant_repeats_bit_for_bit():
    v = variant_number(WIDE4)
    gen = torch.Generator(device="cuda").manual_seed(6)
    X = (torch.rand((770, 1000), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    Y = (torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1).to(torch.bfloat16)
    say("wide4 repeat")
    first = binding.gemm16(X, Y, variant=v)
    second = binding.gemm16(X, Y, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(first, second)


def test_misaligned_operands_fall_back_correctly():
    v = variant_number(WIDE4)
    say("wide4 misaligned fallback")
    C, ref, _ = run("bf16", "N", "N", 300, 520, 136, "int", [4, 5, 6], offset=1, pad=(3, 5, 2), variant=v)
    check_exact(C.view, ref, "misaligned fallback")
    check_padding_untouched(C)
