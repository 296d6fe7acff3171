"""The mixed-precision product (gemm_mixed): bfloat16 / binary16 inputs,
binary32 accumulation, against the 16-bit oracle.

Acceptance as for the fp32 product, against the exact product of the 16-bit
values: integer inputs bit exact, otherwise |C - C_ref| <= 1e-5 S.  Besides,
against the binary32 data before rounding, the error stays within the
rounding of the inputs: |C - C32| <= (2u + u^2) S32 + 1e-5 S, u = 2^-8
(bfloat16) or 2^-11 (binary16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_support import TOL, check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

FORMATS = ["bf16", "f16"]
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
EDGE_SHAPES = [
    (1, 1, 1), (2, 3, 5), (7, 7, 7), (1, 300, 13), (300, 1, 13), (15, 17, 33), (33, 31, 64),
    (63, 65, 127), (127, 129, 255), (257, 255, 1009), (33, 1009, 7), (511, 257, 65), (520, 530, 64),
]


class MixedProblem:
    """16-bit operands in padded device buffers, a sentinel-filled C."""

    def __init__(self, fmt, A: inputs.Padded, B: inputs.Padded, ldc: int, c_offset: int = 0):
        self.fmt, self.A, self.B = fmt, A, B
        self.M, self.K, self.N = A.rows, A.cols, B.cols
        self.ldc, self.c_offset = ldc, c_offset
        self.A_dev = torch.from_numpy(A.buf.view(np.int16)).cuda()
        self.B_dev = torch.from_numpy(B.buf.view(np.int16)).cuda()
        self.C_init = inputs.padded_output(self.M, self.N, ldc, c_offset)
        self.C_dev = torch.from_numpy(self.C_init.buf).cuda()

    def args(self):
        return (self.fmt, self.M, self.N, self.K,
                self.A_dev.data_ptr() + 2 * self.A.offset, self.A.ld,
                self.B_dev.data_ptr() + 2 * self.B.offset, self.B.ld,
                self.C_dev.data_ptr() + 4 * self.c_offset, self.ldc)

    def run(self, variant=None, stream=None) -> inputs.Padded:
        self.C_dev.copy_(torch.from_numpy(self.C_init.buf))
        torch.cuda.synchronize()
        if variant is None:
            binding.gemm_mixed(*self.args(), stream=stream)
        else:
            binding.gemm_mixed_variant(variant, *self.args(), stream=stream)
        torch.cuda.synchronize()
        return inputs.Padded(self.C_dev.cpu().numpy(), self.M, self.N, self.ldc, self.c_offset)


def make(fmt, M, N, K, dist, gen, offset=0, pad=(0, 0, 0)):
    A32 = inputs.random_matrix(gen, M, K, dist)
    B32 = inputs.random_matrix(gen, K, N, dist)
    A = inputs.padded16(inputs.to16(A32, fmt), max(K + pad[0], 1), offset, fmt)
    B = inputs.padded16(inputs.to16(B32, fmt), max(N + pad[1], 1), offset, fmt)
    return MixedProblem(fmt, A, B, max(N + pad[2], 1), offset), A32, B32


def check(prob, C, dist, what, ref=None):
    Cref, S = ref if ref is not None else oracle.gemm16(prob.fmt, prob.A.view, prob.B.view, threads=8)
    if dist == "int":
        check_exact(C.view, Cref, what)
    else:
        check_close(C.view, Cref, S, what)
    check_padding_untouched(C)
    return Cref, S


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_edge_shapes(fmt, dist):
    """Ragged shapes on the default path; offset 0 with even leading
    dimensions takes vector loads, offset 1 (2-byte aligned views) and odd
    leading dimensions take element-wise loads."""
    for (M, N, K) in EDGE_SHAPES:
        for offset, pad in ((0, (0, 0, 0)), (0, (6, 2, 3)), (1, (3, 5, 2)), (2, (1, 1, 1))):
            gen = np.random.default_rng([M * 1_000_003 + N * 1009 + K, offset, sum(pad), len(fmt)])
            prob, _, _ = make(fmt, M, N, K, dist, gen, offset, pad)
            say(f"mixed {fmt} {dist} M={M} N={N} K={K} offset={offset} pad={pad}")
            check(prob, prob.run(), dist, f"{fmt} {dist} {M}x{N}x{K} off{offset} pad{pad}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_every_variant(fmt):
    """Every tile configuration on shapes that straddle its tiles, on both
    load paths."""
    for v in range(binding.gemm_mixed_num_variants()):
        for (M, N, K, offset) in ((300, 520, 200, 0), (257, 513, 129, 1), (64, 64, 64, 0), (1, 700, 70, 0)):
            for dist in ("int", "uniform"):
                gen = np.random.default_rng([v, M, N, K, offset, len(fmt)])
                prob, _, _ = make(fmt, M, N, K, dist, gen, offset, (2 * offset, 0, 1))
                say(f"mixed {fmt} variant={v} {binding.gemm_mixed_variant_name(v)} {M}x{N}x{K} off{offset} {dist}")
                check(prob, prob.run(variant=v), dist, f"variant {v} {M}x{N}x{K} {dist}")


SCHED = 8          # the scheduled 4-wave kernel (256 x 256 tiles, K % 8 == 0, N even)
SCHED_SHAPES = [(256, 256, 64), (256, 512, 128), (512, 256, 192), (768, 1024, 320), (1024, 1024, 1024),
                (512, 768, 4160),
                # edge tiles run whole: ragged M (any), ragged N (even; N % 8 = 4
                # or 2: the last row's chunk across the end reads zeros past it)
                (264, 520, 128), (1000, 1000, 1024), (300, 776, 192), (8, 264, 64), (301, 516, 128),
                (257, 1026, 64),
                # K a multiple of 8, the last phase partial: one, two, three and more phases
                (256, 256, 8), (512, 512, 72), (512, 256, 136), (264, 520, 200), (300, 776, 1000)]


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_scheduled_kernel(fmt):
    """The scheduled kernel on shapes it takes: one, two, three and more
    phases (its prologue, tail and main-loop paths), long K, edge tiles
    (rows past M and columns past N copy zeros or feed only unstored C
    entries; the NaN padding of the operands must not reach C) and a last
    phase that reaches past K (its chunks there copy zeros); integer data
    exactly, float data within the bound, and the same bits as the 8-wave
    kernel of configuration 6 (same tiles, same k order)."""
    assert binding.gemm_mixed_variant_name(SCHED) == "mixed256x256_bk64_w4_sched"
    for (M, N, K) in SCHED_SHAPES:
        for dist in ("int", "uniform"):
            gen = np.random.default_rng([M, N, K, len(fmt), len(dist)])
            prob, _, _ = make(fmt, M, N, K, dist, gen)
            say(f"mixed {fmt} scheduled {M}x{N}x{K} {dist}")
            C = prob.run(variant=SCHED)
            check(prob, C, dist, f"scheduled {fmt} {M}x{N}x{K} {dist}")
            ref6 = prob.run(variant=6).view.copy()
            assert np.array_equal(C.view.view(np.uint32), ref6.view(np.uint32)), (fmt, M, N, K, dist)
            del prob


def test_mixed_scheduled_kernel_padded_and_fallback():
    """Padded leading dimensions and ragged M (still taken by the scheduled
    kernel), and shapes it does not take (odd N, K not a multiple of 8,
    2-byte-offset views), which run configuration 6 instead: same bits
    either way."""
    gen = np.random.default_rng(123)
    cases = [(512, 512, 256, 0, (8, 16, 3)), (520, 512, 256, 0, (0, 0, 0)), (512, 512, 204, 0, (0, 0, 0)),
             (512, 512, 256, 1, (2, 2, 2)), (512, 515, 256, 0, (0, 1, 0)), (520, 264, 256, 0, (8, 16, 3))]
    for (M, N, K, offset, pad) in cases:
        prob, _, _ = make("bf16", M, N, K, "uniform", gen, offset, pad)
        say(f"mixed scheduled/fallback {M}x{N}x{K} offset={offset} pad={pad}")
        C = prob.run(variant=SCHED)
        check(prob, C, "uniform", f"scheduled/fallback {M}x{N}x{K}")
        ref6 = prob.run(variant=6).view.copy()
        assert np.array_equal(C.view.view(np.uint32), ref6.view(np.uint32)), (M, N, K, offset, pad)


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_load_paths_agree_bitwise(fmt):
    """The vector and element-wise load paths of one tile configuration sum
    in the same order: the same data at an aligned and at a 2-byte-offset
    address give the same bits, for the configurations the default path
    picks besides the k-split one (64 x 64, 128 x 128 with direct copies, the
    scheduled 256 x 256).  The k-split configuration's 16-byte copies need
    4-byte alignment; a misaligned call given to it runs the element-wise
    64 x 64 kernel, whose order differs: the default is checked against the
    oracle at both addresses instead."""
    names = ("mixed64x64_bk64_w1x2", "mixed128x128_bk64_w2x2_directAB", "mixed256x256_bk64_w4_sched")
    configs = [v for v in range(binding.gemm_mixed_num_variants()) if binding.gemm_mixed_variant_name(v) in names]
    assert len(configs) == 3
    for (M, N, K) in ((520, 530, 200), (1000, 1000, 1000), (300, 2100, 776)):
        gen = np.random.default_rng([M, N, K, 7, len(fmt)])
        A32 = inputs.random_matrix(gen, M, K, "uniform")
        B32 = inputs.random_matrix(gen, K, N, "uniform")
        probs = []
        for offset in (0, 1):
            A = inputs.padded16(inputs.to16(A32, fmt), K, offset, fmt)
            B = inputs.padded16(inputs.to16(B32, fmt), N, offset, fmt)
            probs.append(MixedProblem(fmt, A, B, N))
        for v in configs:
            say(f"mixed {fmt} load paths {M}x{N}x{K} variant={v}")
            out = [pr.run(variant=v).view.copy() for pr in probs]
            assert np.array_equal(out[0].view(np.uint32), out[1].view(np.uint32)), (fmt, M, N, K, v)
        say(f"mixed {fmt} load paths {M}x{N}x{K} default")
        ref, S = oracle.gemm16(fmt, probs[0].A.view, probs[0].B.view, threads=8)
        for pr in probs:
            check_close(pr.run().view, ref, S, f"{fmt} {M}x{N}x{K} default, offset {pr.A.offset}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_workloads_full(fmt):
    """square256 and square1000 against the full 16-bit oracle, integer and
    float data; the float result also against the binary32 data before
    rounding, within the inputs' rounding."""
    for name in ("square256", "square1000"):
        w = inputs.WORKLOADS[name]
        for dist in ("int", w.dist):
            A, B, A32, B32 = inputs.operands16(w, fmt, dist)
            prob = MixedProblem(fmt, A, B, w.ldc, w.offset)
            say(f"mixed {fmt} workload {name} {dist}")
            C = prob.run()
            check(prob, C, dist, f"{name} {fmt} {dist}")
            if dist != "int":
                C32, S32 = oracle.gemm(A32, B32, threads=8)
                _, S16 = oracle.gemm16(fmt, A.view, B.view, threads=8)
                u = UNIT_ROUNDOFF[fmt]
                err = np.abs(C.view.astype(np.float64) - C32)
                assert np.all(err <= (2 * u + u * u) * S32 + TOL * S16), (name, fmt, err.max())


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", ["square4096", "rect8192x4096x2048_padded", "square8192"])
def test_mixed_workloads_sampled(fmt, name):
    """The large workloads (the rect one through 2-byte-offset views, so on
    element-wise loads) on sampled entries plus edge entries, integer data
    exactly, float data within the bound."""
    w = inputs.WORKLOADS[name]
    for dist in ("int", w.dist):
        A, B, _, _ = inputs.operands16(w, fmt, dist)
        prob = MixedProblem(fmt, A, B, w.ldc, w.offset)
        say(f"mixed {fmt} workload {name} {dist} (sampled)")
        C = prob.run()
        ii, jj = inputs.sample_pairs(w.M, w.N, 4096, inputs.rng(w.index, 4))
        c, s = oracle.gemm16_entries(fmt, A.view, B.view, ii, jj)
        got = C.view[ii, jj]
        if dist == "int":
            check_exact(got, c, f"{name} {fmt} int sample")
        else:
            check_close(got, c, s, f"{name} {fmt} sample")
        check_padding_untouched(C)
        del prob
        torch.cuda.empty_cache()


def test_mixed_degenerate_and_repeat():
    """K = 0 writes +0; empty M or N is a no-op; repeated calls and a side
    stream give the same bits; a long K stays exact on integers."""
    gen = np.random.default_rng(99)
    for fmt in FORMATS:
        prob, _, _ = make(fmt, 70, 90, 0, "int", gen)
        C = prob.run()
        assert np.all(C.view == 0) and not np.any(np.signbit(C.view))
        check_padding_untouched(C)
        binding.gemm_mixed(fmt, 0, 5, 5, None, 5, None, 5, None, 5)
        binding.gemm_mixed(fmt, 5, 0, 5, None, 5, None, 1, None, 1)
        prob, _, _ = make(fmt, 300, 260, 1000, "uniform", gen)
        first = prob.run().view.copy()
        side = torch.cuda.Stream()
        again = prob.run(stream=side).view.copy()
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
        prob, _, _ = make(fmt, 40, 70, 70001, "int", gen)
        say(f"mixed {fmt} long K=70001")
        check(prob, prob.run(), "int", f"{fmt} long K")


def test_mixed_tensor_form():
    """gemm16() on torch bfloat16/float16 tensors, views with a leading
    dimension included, matches the oracle."""
    gen = np.random.default_rng(5)
    for fmt, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        A32 = inputs.random_matrix(gen, 130, 77, "uniform")
        B32 = inputs.random_matrix(gen, 77, 150, "uniform")
        Ab, Bb = inputs.to16(A32, fmt), inputs.to16(B32, fmt)
        big = torch.zeros((130, 80), dtype=torch.int16)
        big[:, :77] = torch.from_numpy(Ab.view(np.int16))
        A_t = big.cuda().view(dt)[:, :77]
        B_t = torch.from_numpy(Bb.view(np.int16)).cuda().view(dt)
        C = binding.gemm16(A_t, B_t)
        torch.cuda.synchronize()
        Cref, S = oracle.gemm16(fmt, Ab, Bb)
        check_close(C.cpu().numpy(), Cref, S, f"tensor form {fmt}")
