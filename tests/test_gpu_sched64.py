"""64 x 64 tiles of 2 x 2 waves, each one 32 x 32 block over the whole K
(gemm_f32_tile64_kernel: diagnostic variant mfma64x64_bk32_w2x2_sched, three
LDS stages, the default for short-K shapes with several tiles per CU; and
its four- and two-stage forms) against the fp32 oracle: exact on integer
inputs, within 1e-5 S on uniform ones.

The last phase skips its 8-deep steps that lie wholly at k >= K, so the
shapes take every count of k in the last phase that a multiple of 4 allows
(4 .. 32), with one phase in all and with several, and phase counts that
leave every stage count's unrolled loop a tail of each length; edge tiles on
both sides; offset views whose pad words are NaN; a second call with the
same bits, and the same bits from every stage count; problems it does not
take (K % 4 != 0) handed to configuration 20's kernels; every op pair
through gemm_f32_op where it is the default."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs
from test_gpu_ksplit import variant_number

pytestmark = pytest.mark.gpu

S64 = "mfma64x64_bk32_w2x2_sched"
S64_4 = "mfma64x64_bk32_w2x2_4stage"        # the same tiles, four LDS stages
S64_2 = "mfma64x64_bk32_w2x2_2stage"        # two

# (M, N, K) and the k in the last phase: 4 (one phase), 8, 12, 20, 4 (two
# phases), 28, 24, 8 (32 phases), 32 (16 phases)
SHAPES = [(64, 64, 4), (100, 136, 8), (64, 128, 12), (136, 200, 20), (200, 64, 36), (580, 520, 60),
          (128, 192, 88), (300, 392, 1000), (1000, 1000, 512)]


def run_variant(M, N, K, dist, seed, name=S64):
    gen = np.random.default_rng(seed)
    A = inputs.padded(inputs.random_matrix(gen, M, K, dist), K + 3, 1)
    B = inputs.padded(inputs.random_matrix(gen, K, N, dist), N + 5, 1)
    Cref, S = oracle.gemm(A.view, B.view, threads=8)
    A_dev = torch.from_numpy(A.buf).cuda()
    B_dev = torch.from_numpy(B.buf).cuda()
    C_init = inputs.padded_output(M, N, N + 7, 1)
    C_dev = torch.from_numpy(C_init.buf).cuda()
    binding.gemm_f32_variant(variant_number(name), M, N, K, A_dev.data_ptr() + 4, A.ld, B_dev.data_ptr() + 4,
                             B.ld, C_dev.data_ptr() + 4, N + 7)
    torch.cuda.synchronize()
    return inputs.Padded(C_dev.cpu().numpy(), M, N, N + 7, 1), Cref, S


@pytest.mark.parametrize("name", [S64, S64_2, S64_4])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(dist, name):
    for (M, N, K) in SHAPES:
        say(f"{name} variant {dist} {(M, N, K)}")
        C, Cref, S = run_variant(M, N, K, dist, [M, N, K, dist == "int", 19], name)
        check_padding_untouched(C)
        what = f"{name} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, Cref, what)
        else:
            check_close(C.view, Cref, S, what)


@pytest.mark.parametrize("name", [S64, S64_2, S64_4])
def test_variant_repeats_bit_for_bit(name):
    v = variant_number(name)
    gen = torch.Generator(device="cuda").manual_seed(9)
    X = torch.rand((580, 1000), device="cuda", generator=gen) * 2 - 1
    Y = torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1
    say("sched64 repeat")
    outs = []
    for _ in range(2):
        C = torch.empty((580, 520), device="cuda")
        binding.gemm_f32_variant(v, 580, 520, 1000, X, 1000, Y, 520, C, 520)
        outs.append(C)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("name", [S64, S64_2, S64_4])
def test_fallback_for_k_not_multiple_of_4(name):
    say(f"{name} fallback")
    C, Cref, _ = run_variant(200, 136, 102, "int", [5, 6, 8], name)
    check_padding_untouched(C)
    check_exact(C.view, Cref, f"{name} fallback")


def test_stage_counts_give_the_same_bits():
    """The forms run the same instructions on the same fragments in the same
    order: the same bits."""
    outs = []
    gen = torch.Generator(device="cuda").manual_seed(10)
    X = torch.rand((1000, 1000), device="cuda", generator=gen) * 2 - 1
    Y = torch.rand((1000, 1000), device="cuda", generator=gen) * 2 - 1
    for name in (S64, S64_2, S64_4):
        say(f"{name} same bits")
        C = torch.empty((1000, 1000), device="cuda")
        binding.gemm_f32_variant(variant_number(name), 1000, 1000, 1000, X, 1000, Y, 1000, C, 1000)
        outs.append(C)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def test_default_for_its_shapes():
    for shape in [(3000, 3000, 384), (2048, 3072, 512), (1000, 2000, 500), (1532, 1028, 388)]:
        assert binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(*shape)) == S64, shape


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_op_pairs_full_oracle(ops, dist):
    """Every entry against the oracle, every op pair through gemm_f32_op,
    which runs this kernel at 1532 x 1028 x 388 (edge tiles on both sides,
    4 k in the last phase) and 1000 x 2000 x 500 (20 in the last phase); a
    second call and the op N, N product of transposed copies give the same
    bits."""
    from test_gpu_ksplit import Problem
    op_a, op_b = ops
    for (M, N, K) in [(1532, 1028, 388), (1000, 2000, 500)]:
        prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, len(op_a + op_b), dist == "int", ord(op_b), 64])
        Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
        say(f"sched64 full {op_a}{op_b} {dist} {(M, N, K)}")
        C = prob.run()
        check_padding_untouched(C)
        what = f"{S64} {op_a}{op_b} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, Cref, what)
        else:
            check_close(C.view, Cref, S, what)
        again = prob.run()
        assert np.array_equal(C.view, again.view), what + ": a second call gave other bits"
        assert np.array_equal(C.view, prob.plain_bits()), what + ": bits differ from the op N, N product"
