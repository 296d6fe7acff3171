"""Helpers for the GPU parity tests: device copies of padded operands, calls
through the C ABI, and the acceptance checks.

Acceptance (per output element, compared in binary64):
  * integer-valued inputs: the GPU value equals the oracle's sum rounded to
    binary32, exactly (every product and partial sum is an integer below 2^24,
    so any summation order is exact);
  * otherwise |C_gpu - C| <= 1e-5 * sum_k |A_ik B_kj|, and an entry whose
    scale is 0 must be exactly 0;
  * every word of C outside the M x N window keeps its sentinel bits, and A/B
    padding (NaN) never reaches a result.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from shared_memory_tiled_amd import binding, inputs

TOL = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceProblem:
    """One product's operands on the GPU, in padded buffers."""

    def __init__(self, A: inputs.Padded, B: inputs.Padded, ldc: int, c_offset: int = 0):
        assert A.cols == B.rows
        self.M, self.K, self.N = A.rows, A.cols, B.cols
        self.A, self.B = A, B
        self.ldc, self.c_offset = ldc, c_offset
        self.A_dev = torch.from_numpy(A.buf).to("cuda")
        self.B_dev = torch.from_numpy(B.buf).to("cuda")
        self.C_init = inputs.padded_output(self.M, self.N, ldc, c_offset)
        self.C_dev = torch.from_numpy(self.C_init.buf).to("cuda")

    def args(self):
        return (self.M, self.N, self.K,
                self.A_dev.data_ptr() + 4 * self.A.offset, self.A.ld,
                self.B_dev.data_ptr() + 4 * self.B.offset, self.B.ld,
                self.C_dev.data_ptr() + 4 * self.c_offset, self.ldc)

    def reset_c(self):
        self.C_dev.copy_(torch.from_numpy(self.C_init.buf))
        torch.cuda.synchronize()

    def run(self, variant=None, stream=None, reset=True):
        if reset:
            self.reset_c()
        if variant is None:
            binding.gemm_f32(*self.args(), stream=stream)
        else:
            binding.gemm_f32_variant(variant, *self.args(), stream=stream)
        torch.cuda.synchronize()

    def result(self) -> inputs.Padded:
        buf = self.C_dev.cpu().numpy()
        return inputs.Padded(buf, self.M, self.N, self.ldc, self.c_offset)


def check_padding_untouched(C: inputs.Padded) -> None:
    bits = C.buf.view(np.uint32)
    s = inputs.C_SENTINEL_BITS
    n = C.rows * C.ld
    assert np.all(bits[:C.offset] == s), "C words before the view were written"
    assert np.all(bits[C.offset + n:] == s), "C guard words after the view were written"
    if C.rows and C.ld > C.cols:
        pad = bits[C.offset:C.offset + n].reshape(C.rows, C.ld)[:, C.cols:]
        assert np.all(pad == s), "C padding between N and ldc was written"


def check_close(got: np.ndarray, ref: np.ndarray, scale: np.ndarray, what: str, tol=TOL) -> None:
    g = got.astype(np.float64)
    err = np.abs(g - ref)
    ok = err <= tol * scale
    ok &= np.where(scale == 0, g == 0, True)
    if not np.all(ok):
        bad = np.argwhere(~ok)
        idx = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} entries outside |err| <= {tol}*S; first at {idx}: "
            f"gpu={g[idx]!r} oracle={ref[idx]!r} S={scale[idx]!r}")


def check_exact(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    want = ref.astype(np.float32)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        idx = tuple(bad[0]) if len(bad) else None
        raise AssertionError(f"{what}: {len(bad)} entries differ from the exact integer result; "
                             f"first at {idx}: gpu={got[idx]!r} oracle={want[idx]!r}")
