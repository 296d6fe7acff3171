"""reduce_sum_f32_variant_noalloc (the reduction with its partials in the
library's fixed per-device scratch) against reduce_sum_f32_variant (the same
reduction with a workspace from the caller), through the C ABI.

Two calls in a row per variant, the second on a smaller input, so the second
runs over scratch still holding the first call's partials: the deterministic
variants (0, 1, 2, 4) must give the workspace entry point's bits both times,
and the atomic variant (3) its error bound against the oracle.  Both entry
points run the same kernels in the same order, so equal bits are the bar.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_support import say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
# (first n, second n): the second smaller, with ragged tails; the first sizes
# fill most of the scratch for the tree versions (about 4 n / 255 bytes).
SIZES = {0: (60_000_001, 1_000_003), 1: (60_000_001, 65_537), 2: (33_554_433, 257),
         3: (5_000_003, 4_097), 4: (200_000_003, 1_000_003)}


def with_workspace(v: int, x: torch.Tensor, n: int) -> float:
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    wsb = binding.reduce_sum_f32_workspace_size(v, n)
    ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device="cuda")
    binding.reduce_sum_f32_variant(v, n, x, out, ws, wsb)
    torch.cuda.synchronize()
    return float(out.cpu().numpy()[0])


def without_workspace(v: int, x: torch.Tensor, n: int) -> float:
    out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    binding.reduce_sum_f32_variant_noalloc(v, n, x, out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return float(out.cpu().numpy()[0])


@pytest.mark.parametrize("variant", sorted(SIZES))
def test_noalloc_matches_workspace_entry_point(variant):
    for call, n in enumerate(SIZES[variant]):
        gen = inputs.rng(90 + variant, call)
        x_host = inputs.random_matrix(gen, 1, n, "uniform").reshape(-1)
        x = torch.from_numpy(x_host).cuda()
        say(f"noalloc reduce variant={variant} call={call} n={n}")
        got = without_workspace(variant, x, n)
        ref = with_workspace(variant, x, n)
        if variant == 3:
            exact, scale = oracle.reduce_sum(x_host)
            bound = (8 + math.ceil(n / 256) + 1) * U * scale * 1.000001
            assert abs(got - exact) <= bound, (n, got, exact, bound)
            assert abs(ref - exact) <= bound, (n, ref, exact, bound)
        else:
            assert got == ref, (variant, n, got, ref)
        del x


def test_noalloc_integer_sums_exact_and_empty():
    """Integer data (every partial exact) gives the oracle's sum on every
    variant; n = 0 writes +0; a rejected size leaves *out untouched."""
    n = 3_000_017
    x_host = np.random.default_rng(77).integers(-1, 2, n).astype(np.float32)
    exact, _ = oracle.reduce_sum(x_host)
    x = torch.from_numpy(x_host).cuda()
    for v in range(binding.reduce_sum_f32_num_variants()):
        say(f"noalloc reduce integer variant={v} n={n}")
        assert without_workspace(v, x, n) == exact, v
        assert without_workspace(v, x, 0) == 0.0
    out = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemmError) as err:
        binding.reduce_sum_f32_variant_noalloc(0, 2 ** 27, x, out)   # refused before any launch
    assert err.value.status == 12
    torch.cuda.synchronize()
    assert float(out.cpu().numpy()[0]) == 5.0
