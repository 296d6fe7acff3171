"""The CPU oracle against its pins (no GPU needed)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(lib, check):
    check(lib)


def test_k_zero_and_empty(lib):
    A = np.zeros((4, 0), np.float32)
    B = np.zeros((0, 6), np.float32)
    C, S = oracle.gemm(A, B, lib=lib)
    assert C.shape == (4, 6) and np.all(C == 0) and not np.any(np.signbit(C)) and np.all(S == 0)
    C, S = oracle.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 3), np.float32), lib=lib)
    assert C.shape == (0, 3)


def test_rejects_bad_arguments(lib):
    A = np.ones((3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm(A, np.ones((5, 2), np.float32), lib=lib)
    with pytest.raises(ValueError):
        oracle.gemm_entries(A, np.ones((4, 2), np.float32), [3], [0], lib=lib)
    with pytest.raises(ValueError):
        oracle.tiled_traffic(4, 4, 4, 0, 4, 4, lib=lib)
