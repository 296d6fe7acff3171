"""Every reduction variant against the oracle's binary64 sum: exact on small
integers, within its summation-error bound on floats; deterministic variants
repeat bit for bit."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_support import say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

VARIANTS = list(range(binding.reduce_sum_f32_num_variants()))
U = 2.0 ** -24


def chain_bound(variant: int, n: int) -> float:
    """Longest sequential chain + tree depth of each variant's summation
    order (see reduce.hip), the factor of 2^-24 sum|x| in its error bound."""
    if n <= 1:
        return 1.0
    if variant in (0, 1, 2):                 # trees of 256 per pass
        passes = max(1, math.ceil(math.log(n, 256) - 1e-12))
        return 8 * passes + 1
    if variant == 3:                         # tree of 256, then atomics block by block
        return 8 + math.ceil(n / 256) + 1
    # grid_vec: 2048 blocks of 256 threads; per thread a sequential run of
    # chunks (+1 for the tail), 2 + 6 + 2 levels to the block partial, then
    # 8 partials per thread, 6 + 2 levels in the second pass
    stride = 2048 * 256
    return math.ceil(n / 4 / stride) + 1 + 10 + 16


def gpu_sum(x: np.ndarray, variant, dev_x=None) -> float:
    xt = torch.from_numpy(x).cuda() if dev_x is None else dev_x
    out = binding.reduce_sum(xt, variant=variant)
    torch.cuda.synchronize()
    return float(out.cpu().numpy()[0])


SIZES = [0, 1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1000, 4096, 65535, 65536, 65537, 1_000_003]


def vname(v):
    return "default" if v is None else f"{v}-{binding.reduce_sum_f32_variant_name(v)}"


@pytest.mark.parametrize("variant", [None] + VARIANTS, ids=vname)
def test_reduce_sizes(variant):
    for n in SIZES:
        for dist in ("int", "uniform"):
            gen = np.random.default_rng([n, 0 if dist == "int" else 1])
            if dist == "int":
                x = gen.integers(-1, 2, n).astype(np.float32)
            else:
                x = inputs.random_matrix(gen, 1, n, "uniform").reshape(-1)
            ref, scale = oracle.reduce_sum(x)
            say(f"reduce variant={vname(variant)} n={n} dist={dist}")
            got = gpu_sum(x, variant)
            v = 4 if variant is None else variant
            if dist == "int":
                assert got == ref, (variant, n, got, ref)
            else:
                assert abs(got - ref) <= chain_bound(v, n) * U * scale * 1.000001, (variant, n, got, ref, scale)
            if n == 0:
                assert got == 0.0 and not math.copysign(1.0, got) < 0


def test_reduce_pages_example_and_determinism():
    """The page's 2^24 inputs (values -1, 0, 1: every partial sum exact), on
    every variant; then uniform values, where each deterministic variant
    repeats itself bit for bit."""
    n = 2 ** 24
    gen = np.random.default_rng(2024)
    xi = gen.integers(-1, 2, n).astype(np.float32)
    ref, _ = oracle.reduce_sum(xi)
    dev = torch.from_numpy(xi).cuda()
    for v in VARIANTS:
        say(f"2^24 integer sum variant={vname(v)}")
        assert gpu_sum(xi, v, dev) == ref, v
    xf = inputs.random_matrix(gen, 1, n, "uniform").reshape(-1)
    ref, scale = oracle.reduce_sum(xf)
    dev = torch.from_numpy(xf).cuda()
    for v in VARIANTS:
        say(f"2^24 float sum variant={vname(v)}")
        a, b = gpu_sum(xf, v, dev), gpu_sum(xf, v, dev)
        assert abs(a - ref) <= chain_bound(v, n) * U * scale * 1.000001, (v, a, ref)
        if v != 3:
            assert a == b, v


def test_reduce_large_offset_view():
    """A 2^28 + 3 float array read through a pointer 4 bytes past an aligned
    address (the 128-bit loads of the default variant are dword aligned)."""
    n = 2 ** 28 + 3
    gen = np.random.default_rng(7)
    x = np.empty(n + 1, np.float32)
    x[1:] = inputs.random_matrix(gen, 1, n, "uniform").reshape(-1)
    x[0] = np.nan
    ref, scale = oracle.reduce_sum(x[1:])
    dev = torch.from_numpy(x).cuda()
    out = torch.empty(1, device="cuda")
    ws_bytes = binding.reduce_sum_f32_workspace_size(4, n)
    ws = torch.empty(ws_bytes // 4, device="cuda")
    say("reduce 2^28+3 offset view")
    binding.reduce_sum_f32(n, dev.data_ptr() + 4, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = float(out.cpu()[0])
    assert abs(got - ref) <= chain_bound(4, n) * U * scale * 1.000001, (got, ref, scale)
