"""The small-product kernels (16 x 16 or 32 x 32 output tiles whose k groups
are split over the waves of a block, operands loaded straight into
registers) against the oracle: exact on integer inputs, within 1e-5 S on
uniform ones, on ragged shapes, offset views with padded leading dimensions,
K = 0 and single rows or columns; C padding untouched."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

CONFIGS = ["mfma16x16_w4_small", "mfma32x32_w4_small", "mfma16x16_w8_small"]
SHAPES = [(1, 1, 1), (16, 16, 16), (17, 15, 33), (31, 33, 3), (256, 256, 256), (255, 257, 250),
          (100, 37, 1000), (33, 1, 5), (1, 300, 17), (64, 64, 0), (48, 80, 4099), (200, 120, 64)]


def variant_number(name):
    for d in range(binding.gemm_f32_num_diagnostic_variants()):
        if binding.gemm_f32_variant_name(binding.DIAGNOSTIC_BASE + d) == name:
            return binding.DIAGNOSTIC_BASE + d
    raise KeyError(name)


def run_variant(v, A, B, ldc, offset):
    M, K, N = A.rows, A.cols, B.cols
    C0 = inputs.padded_output(M, N, ldc, offset)
    a, b, c = (torch.from_numpy(x.buf).cuda() for x in (A, B, C0))
    binding.gemm_f32_variant(v, M, N, K, a.data_ptr() + 4 * A.offset, A.ld, b.data_ptr() + 4 * B.offset, B.ld,
                             c.data_ptr() + 4 * offset, ldc)
    torch.cuda.synchronize()
    return inputs.Padded(c.cpu().numpy(), M, N, ldc, offset)


@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_small_kernel_against_oracle(config, dist):
    v = variant_number(config)
    for (M, N, K) in SHAPES:
        for offset, pad in ((0, 0), (1, 3)):
            gen = np.random.default_rng([M, N, K, offset, 7])
            A = inputs.padded(inputs.random_matrix(gen, M, K, dist), max(K + pad, 1), offset)
            B = inputs.padded(inputs.random_matrix(gen, K, N, dist), max(N + pad, 1), offset)
            say(f"small config={config} dist={dist} M={M} N={N} K={K} offset={offset}")
            C = run_variant(v, A, B, N + pad, offset)
            ref, S = oracle.gemm(A.view, B.view, threads=8)
            if dist == "int":
                check_exact(C.view, ref, f"{config} {M}x{N}x{K}")
            else:
                check_close(C.view, ref, S, f"{config} {M}x{N}x{K}")
            if K == 0:
                assert np.all(C.view == 0) and not np.any(np.signbit(C.view))
            check_padding_untouched(C)


@pytest.mark.parametrize("config", CONFIGS)
def test_small_kernel_repeats_bit_for_bit(config):
    """Fixed k order (groups by wave, waves added in order): a second call
    gives the same bits."""
    v = variant_number(config)
    gen = np.random.default_rng(11)
    A = inputs.padded(inputs.random_matrix(gen, 300, 700, "uniform"), 700)
    B = inputs.padded(inputs.random_matrix(gen, 700, 260, "uniform"), 260)
    first = run_variant(v, A, B, 260, 0).view.copy()
    assert np.array_equal(first.view(np.uint32), run_variant(v, A, B, 260, 0).view.view(np.uint32))
