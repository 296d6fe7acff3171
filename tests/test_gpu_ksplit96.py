"""96 x 96 tiles whose four waves each run the whole tile over every fourth
16-deep phase (diagnostic variant mfma96x96_bk16_w1x1_k4_sched, the
default for the shapes its tiles fill best) against the fp32 oracle: exact
on integer inputs, within 1e-5 S on uniform ones.

Through the variant (op N, N): one phase in all (three waves without a
phase), K % 16 = 4 (phase 0 reaching below k = 0), one phase per wave (an
odd count: a position copying zeros), two to sixteen phases a wave, edge
tiles on both sides, offset views whose pad words are NaN, a second call
with the same bits, and problems it does not take (K % 4 != 0) handed to
the 64 x 64 k-split tiles."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs
from test_gpu_ksplit import variant_number

pytestmark = pytest.mark.gpu

KS96 = "mfma96x96_bk16_w1x1_k4_sched"

# (M, N, K): K = 4 and 16: one phase in all; 64: one per wave; 100: wave 0
# two (K % 16 = 4); 388: wave 0 seven; 1000: sixteen a wave (K % 16 = 8);
# edge tiles (96 does not divide 200, 136, 580, 520, 1000, 300)
SHAPES = [(96, 96, 4), (200, 136, 16), (96, 192, 64), (200, 136, 100), (580, 520, 388), (300, 392, 1000),
          (1000, 1000, 512)]


def run_variant(M, N, K, dist, seed):
    gen = np.random.default_rng(seed)
    A = inputs.padded(inputs.random_matrix(gen, M, K, dist), K + 3, 1)
    B = inputs.padded(inputs.random_matrix(gen, K, N, dist), N + 5, 1)
    Cref, S = oracle.gemm(A.view, B.view, threads=8)
    A_dev = torch.from_numpy(A.buf).cuda()
    B_dev = torch.from_numpy(B.buf).cuda()
    C_init = inputs.padded_output(M, N, N + 7, 1)
    C_dev = torch.from_numpy(C_init.buf).cuda()
    binding.gemm_f32_variant(variant_number(KS96), M, N, K, A_dev.data_ptr() + 4, A.ld, B_dev.data_ptr() + 4,
                             B.ld, C_dev.data_ptr() + 4, N + 7)
    torch.cuda.synchronize()
    return inputs.Padded(C_dev.cpu().numpy(), M, N, N + 7, 1), Cref, S


@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_variant_against_oracle(dist):
    for (M, N, K) in SHAPES:
        say(f"ksplit96 variant {dist} {(M, N, K)}")
        C, Cref, S = run_variant(M, N, K, dist, [M, N, K, dist == "int", 17])
        check_padding_untouched(C)
        what = f"{KS96} {dist} {(M, N, K)}"
        if dist == "int":
            check_exact(C.view, Cref, what)
        else:
            check_close(C.view, Cref, S, what)


def test_variant_repeats_bit_for_bit():
    v = variant_number(KS96)
    gen = torch.Generator(device="cuda").manual_seed(8)
    X = torch.rand((580, 1000), device="cuda", generator=gen) * 2 - 1
    Y = torch.rand((1000, 520), device="cuda", generator=gen) * 2 - 1
    say("ksplit96 repeat")
    outs = []
    for _ in range(2):
        C = torch.empty((580, 520), device="cuda")
        binding.gemm_f32_variant(v, 580, 520, 1000, X, 1000, Y, 520, C, 520)
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_fallback_for_k_not_multiple_of_4():
    say("ksplit96 fallback")
    C, Cref, _ = run_variant(200, 136, 102, "int", [5, 6, 7])
    check_padding_untouched(C)
    check_exact(C.view, Cref, f"{KS96} fallback")


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def test_default_for_its_shapes():
    for shape in [(1536, 1536, 1536), (1532, 1528, 1540), (3072, 3072, 3072), (4608, 4608, 4608),
                  (7168, 7168, 7168)]:
        assert binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(*shape)) == KS96, shape


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("dist", ["int", "uniform"])
def test_op_pairs_full_oracle(ops, dist):
    """Every entry against the oracle, every op pair through gemm_f32_op,
    which runs this kernel at 1532 x 1528 x 1540 (16 x 16 tiles with ragged
    edges, K % 16 = 4); a second call and the op N, N product of transposed
    copies give the same bits."""
    from test_gpu_ksplit import Problem
    op_a, op_b = ops
    M, N, K = 1532, 1528, 1540
    prob = Problem(op_a, op_b, M, N, K, dist, [M, N, K, len(op_a + op_b), dist == "int", ord(op_b), 96])
    Cref, S = oracle.gemm(prob.A.view, prob.B.view, op_a=op_a, op_b=op_b, threads=8)
    say(f"ksplit96 full {op_a}{op_b} {dist}")
    C = prob.run()
    check_padding_untouched(C)
    what = f"{KS96} {op_a}{op_b} {dist}"
    if dist == "int":
        check_exact(C.view, Cref, what)
    else:
        check_close(C.view, Cref, S, what)
    again = prob.run()
    assert np.array_equal(C.view, again.view), what + ": a second call gave other bits"
    assert np.array_equal(C.view, prob.plain_bits()), what + ": bits differ from the op N, N product"


@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_op_pairs_sampled(ops):
    """4600 x 4604 x 4608 (ragged edges, 9 rounds), views one float into
    their padded allocations: sampled entries against the oracle."""
    from test_gpu_ksplit import Problem
    op_a, op_b = ops
    M, N, K = 4600, 4604, 4608
    prob = Problem(op_a, op_b, M, N, K, "uniform", [M, N, K, len(op_a + op_b), 97], 1, (3, 1, 5))
    ii, jj = inputs.sample_pairs(M, N, 4096, np.random.default_rng([M, N, K, 12]))
    cref, sref = oracle.gemm_entries(prob.A.view, prob.B.view, ii, jj, op_a=op_a, op_b=op_b)
    say(f"ksplit96 sampled {op_a}{op_b}")
    C = prob.run()
    check_padding_untouched(C)
    check_close(C.view[ii, jj], cref, sref, f"{KS96} sampled {op_a}{op_b}")
    assert np.all(np.isfinite(C.view))
