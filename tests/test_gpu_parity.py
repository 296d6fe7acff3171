"""Parity of every kernel of the ladder with the CPU oracle, through the C ABI.

Small and medium problems are checked element by element in full; the large
workloads are checked on a seeded sample of entries (plus edge entries), on
their padding, and on properties that hold at any size.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_support import DeviceProblem, check_close, check_exact, check_padding_untouched, say
from shared_memory_tiled_amd import binding, inputs

pytestmark = pytest.mark.gpu

RUNGS = [0, 1, 2, 3]
DIAGNOSTICS = [binding.DIAGNOSTIC_BASE + d for d in range(binding.gemm_f32_num_diagnostic_variants())]
VARIANTS = RUNGS + DIAGNOSTICS


def vname(v):
    return "default" if v is None else f"{v}-{binding.gemm_f32_variant_name(v)}"


# Shapes around the tile edges of every kernel (16, 32, 64, 128, 256), primes,
# K not a multiple of 4, and degenerate vectors.
EDGE_SHAPES = [
    (1, 1, 1), (1, 1, 7), (2, 3, 5), (7, 7, 7), (1, 300, 13), (300, 1, 13),
    (15, 17, 33), (31, 33, 63), (63, 65, 127), (65, 63, 3), (127, 129, 255),
    (129, 127, 257), (255, 257, 129), (257, 255, 1009), (33, 1009, 7),
    (257, 511, 65), (511, 257, 33), (300, 200, 2),
    (4097, 31, 40), (17, 4099, 33), (520, 530, 64),
]


@functools.lru_cache(maxsize=None)
def edge_case(shape, dist, offset):
    M, N, K = shape
    gen = np.random.default_rng([M * 1_000_003 + N * 1009 + K, offset, 0 if dist == "int" else 1])
    lda, ldb, ldc = K + 3 * offset, N + 5 * offset, N + 7 * offset
    A = inputs.padded(inputs.random_matrix(gen, M, K, dist), lda, offset)
    B = inputs.padded(inputs.random_matrix(gen, K, N, dist), ldb, offset)
    C, S = oracle.gemm(A.view, B.view, threads=8)
    return A, B, ldc, C, S


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("variant", VARIANTS, ids=vname)
def test_edge_shapes(variant, dist):
    for shape in EDGE_SHAPES:
        for offset in (0, 1):
            A, B, ldc, Cref, S = edge_case(shape, dist, offset)
            prob = DeviceProblem(A, B, ldc, offset)
            say(f"variant={vname(variant)} dist={dist} shape={shape} offset={offset}")
            prob.run(variant)
            C = prob.result()
            check_padding_untouched(C)
            what = f"{vname(variant)} {dist} {shape} offset {offset}"
            if dist == "int":
                check_exact(C.view, Cref, what)
            else:
                check_close(C.view, Cref, S, what)


@functools.lru_cache(maxsize=None)
def workload_case(name, dist):
    w = inputs.WORKLOADS[name]
    A, B = inputs.operands(w, dist=dist)
    C, S = oracle.gemm(A.view, B.view, threads=8)
    return w, A, B, C, S


@pytest.mark.parametrize("dist", ["int", None])
@pytest.mark.parametrize("name", ["square256", "square1000"])
@pytest.mark.parametrize("variant", [None] + VARIANTS, ids=vname)
def test_workload_full(variant, name, dist):
    w, A, B, Cref, S = workload_case(name, dist)
    prob = DeviceProblem(A, B, w.ldc, w.offset)
    say(f"variant={vname(variant)} workload={name} dist={dist or w.dist}")
    prob.run(variant)
    C = prob.result()
    check_padding_untouched(C)
    if dist == "int":
        check_exact(C.view, Cref, f"{name} int {vname(variant)}")
    else:
        check_close(C.view, Cref, S, f"{name} {vname(variant)}")
    prob.run(variant)                        # deterministic: same bits again
    assert np.array_equal(prob.result().buf.view(np.uint32), C.buf.view(np.uint32))


def test_rungs_agree():
    """Integer inputs: every variant gives the same bits.  Float inputs: each
    rung is within 2e-5 S of the rung below it (both are within 1e-5 S of the
    exact product)."""
    w, A, B, _, _ = workload_case("square256", "int")
    prob = DeviceProblem(A, B, w.ldc, w.offset)
    base = None
    for v in VARIANTS:
        say(f"int agreement variant={vname(v)}")
        prob.run(v)
        bits = prob.result().view.copy()
        if base is None:
            base = bits
        assert np.array_equal(bits, base), vname(v)
    w, A, B, _, S = workload_case("square1000", None)
    prob = DeviceProblem(A, B, w.ldc, w.offset)
    prev = None
    for v in RUNGS:
        say(f"float ladder variant={vname(v)}")
        prob.run(v)
        cur = prob.result().view.astype(np.float64)
        if prev is not None:
            assert np.all(np.abs(cur - prev) <= 2e-5 * S), f"rung {v} vs rung {v - 1}"
        prev = cur


@pytest.mark.parametrize("variant", VARIANTS, ids=vname)
def test_k_zero_and_empty(variant):
    M, N = 70, 45
    A = inputs.padded(np.zeros((M, 0), np.float32), 1, 1)
    B = inputs.padded(np.zeros((0, N), np.float32), N + 2, 1)
    prob = DeviceProblem(A, B, N + 3, 1)
    say(f"K=0 variant={vname(variant)}")
    prob.run(variant)
    C = prob.result()
    check_padding_untouched(C)
    assert np.all(C.view == 0) and not np.any(np.signbit(C.view))
    for (m, n) in ((0, 5), (5, 0)):
        A = inputs.padded(np.ones((m, 4), np.float32), 4)
        B = inputs.padded(np.ones((4, n), np.float32), max(n, 1))
        prob = DeviceProblem(A, B, max(n, 1))
        prob.run(variant)
        C = prob.result()
        assert np.all(C.buf.view(np.uint32) == inputs.C_SENTINEL_BITS)


@pytest.mark.parametrize("variant", VARIANTS, ids=vname)
def test_long_k(variant):
    """Many phases: exact integer sums up to 4K < 2^24."""
    gen = np.random.default_rng(77)
    M, N, K = 40, 72, 70001
    A = inputs.padded(inputs.random_matrix(gen, M, K, "int"), K + 1, 1)
    B = inputs.padded(inputs.random_matrix(gen, K, N, "int"), N, 0)
    Cref, _ = oracle.gemm(A.view, B.view, threads=8)
    prob = DeviceProblem(A, B, N)
    say(f"long K variant={vname(variant)}")
    prob.run(variant)
    check_exact(prob.result().view, Cref, f"long K {vname(variant)}")


def test_side_stream_and_tensor_api():
    """The stream argument is honoured, and the tensor form passes offset views."""
    w, A, B, Cref, S = workload_case("square1000", None)
    dev = torch.device("cuda")
    a_buf = torch.from_numpy(A.buf).to(dev)
    b_buf = torch.from_numpy(B.buf).to(dev)
    At = a_buf[A.offset:A.offset + A.rows * A.ld].view(A.rows, A.ld)[:, :A.cols]
    Bt = b_buf[B.offset:B.offset + B.rows * B.ld].view(B.rows, B.ld)[:, :B.cols]
    s = torch.cuda.Stream()
    for v in [None] + RUNGS:
        out = torch.full((w.M, w.N + 1), float("nan"), device=dev)[:, 1:]
        say(f"stream/tensor api variant={vname(v)}")
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            binding.gemm(At, Bt, out=out, variant=v)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), Cref, S, f"tensor api {vname(v)}")


# ---------------------------------------------------------- large workloads --

LARGE = ["square4096", "rect8192x4096x2048_padded", "square8192"]


@pytest.mark.parametrize("dist", [None, "int"])
@pytest.mark.parametrize("name", LARGE)
def test_large_workload_sampled(name, dist):
    w = inputs.WORKLOADS[name]
    say(f"generating {name} dist={dist or w.dist}")
    A, B = inputs.operands(w, dist=dist)
    ii, jj = inputs.sample_pairs(w.M, w.N, 4096, inputs.rng(w.index, 4))
    cref, sref = oracle.gemm_entries(A.view, B.view, ii, jj)
    prob = DeviceProblem(A, B, w.ldc, w.offset)
    for v in [None] + RUNGS:
        say(f"variant={vname(v)} workload={name} dist={dist or w.dist}")
        prob.run(v)
        C = prob.result()
        check_padding_untouched(C)
        got = C.view[ii, jj]
        if dist == "int":
            check_exact(got, cref, f"{name} int {vname(v)}")
        else:
            check_close(got, cref, sref, f"{name} {vname(v)}")
            assert np.all(np.isfinite(C.view)), "non-finite output (padding leaked?)"


@pytest.mark.parametrize("name", LARGE)
def test_large_workload_scaling_property(name):
    """At full size, every entry: C(2A, B) equals 2 C(A, B) bit for bit
    (power-of-two scaling is exact in any fixed summation order)."""
    w = inputs.WORKLOADS[name]
    say(f"scaling property {name}")
    A, B = inputs.operands(w)
    A2 = inputs.Padded(A.buf * np.float32(2.0), A.rows, A.cols, A.ld, A.offset)
    p1 = DeviceProblem(A, B, w.ldc, w.offset)
    p2 = DeviceProblem(A2, B, w.ldc, w.offset)
    p1.run(None)
    p2.run(None)
    n = w.M * w.ldc
    c1 = p1.C_dev[w.offset:w.offset + n].view(w.M, w.ldc)[:, :w.N]
    c2 = p2.C_dev[w.offset:w.offset + n].view(w.M, w.ldc)[:, :w.N]
    assert torch.equal(c2, 2 * c1)
    assert bool(torch.isfinite(c1).all())
