"""Seeded input generators: distributions, layout, determinism (CPU only)."""
import numpy as np

from shared_memory_tiled_amd import inputs


def test_uniform_grid_and_range():
    X = inputs.random_matrix(inputs.rng(0, 0), 300, 300, "uniform")
    assert X.dtype == np.float32 and X.min() >= -1.0 and X.max() < 1.0
    # 2u - 1 with u on the 2^-24 grid lands on the 2^-23 grid exactly
    assert np.all((X.astype(np.float64) * 2.0**23) % 1.0 == 0.0)


def test_integer_variant_values():
    X = inputs.random_matrix(inputs.rng(0, 2), 200, 200, "int")
    assert set(np.unique(X).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_deterministic_streams():
    a = inputs.random_matrix(inputs.rng(3, 0), 50, 40, "normal")
    b = inputs.random_matrix(inputs.rng(3, 0), 50, 40, "normal")
    c = inputs.random_matrix(inputs.rng(3, 1), 50, 40, "normal")
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_padded_layout():
    dense = np.arange(12, dtype=np.float32).reshape(3, 4)
    p = inputs.padded(dense, ld=7, offset=1)
    assert np.array_equal(p.view, dense)
    assert p.view.ctypes.data - p.buf.ctypes.data == 4
    mask = np.ones(p.buf.shape, bool)
    for r in range(3):
        mask[1 + r * 7: 1 + r * 7 + 4] = False
    assert np.all(np.isnan(p.buf[mask]))
    out = inputs.padded_output(3, 4, 7, 1)
    assert np.all(out.buf.view(np.uint32) == inputs.C_SENTINEL_BITS)


def test_workload_table():
    w = inputs.WORKLOADS["rect8192x4096x2048_padded"]
    assert (w.M, w.N, w.K, w.lda, w.ldb, w.ldc, w.offset) == (8192, 4096, 2048, 2056, 4104, 4104, 1)
    assert inputs.WORKLOADS["square1000"].M % 16 != 0


def test_sample_pairs():
    ii, jj = inputs.sample_pairs(1000, 1000, 4096, inputs.rng(1, 4))
    pairs = set(zip(ii.tolist(), jj.tolist()))
    assert len(pairs) == len(ii) >= 4096
    for c in ((0, 0), (0, 999), (999, 0), (999, 999)):
        assert c in pairs
    assert ii.min() >= 0 and ii.max() < 1000 and jj.min() >= 0 and jj.max() < 1000
    # an entry in the last partial 128-tile row and column
    assert any(i >= 896 for i in ii.tolist()) and any(j >= 896 for j in jj.tolist())


def test_to16_rounds_to_nearest_even():
    """The 16-bit generator rounds binary32 data to the nearest representable
    value, ties to the even pattern; binary16 agrees with numpy's cast."""
    gen = np.random.default_rng(7)
    x = np.concatenate([inputs.random_matrix(gen, 1, 20000, "uniform").ravel(),
                        inputs.random_matrix(gen, 1, 20000, "normal").ravel(),
                        np.float32([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 0.0, -0.0])])
    b = inputs.to16(x, "bf16")
    val = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    up = ((b.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    down = ((b.astype(np.uint32) - 1) << 16).view(np.float32).astype(np.float64)
    err = np.abs(val - x)
    nz = (b & 0x7FFF) != 0                        # the zeros have no pattern below them
    # the neighbouring pattern on x's side of the rounded value (spacings
    # differ on the two sides of a power of two)
    side = np.where(np.sign(x - val) == np.sign(up - val), up, down)
    assert np.all(err[nz] <= np.abs(side - val)[nz] / 2)
    assert np.array_equal(inputs.to16(np.float32([0.0, -0.0]), "bf16"), np.uint16([0x0000, 0x8000]))
    tie = (err == np.abs(side - val) / 2) & (err > 0)
    assert np.all(b[tie] % 2 == 0) and tie.sum() >= 3
    assert np.array_equal(np.signbit(val), np.signbit(x))
    h = inputs.to16(x, "f16")
    assert np.array_equal(h, x.astype(np.float16).view(np.uint16))


def test_operands16_layout():
    w = inputs.WORKLOADS["square256"]
    A, B, A32, B32 = inputs.operands16(w, "bf16", offset=3)
    assert A.buf.dtype == np.uint16 and A.view.shape == (256, 256) and A.offset == 3
    assert np.all(A.buf[:3] == inputs.NAN16["bf16"]) and np.all(A.buf[-inputs.GUARD_WORDS:] == inputs.NAN16["bf16"])
    assert np.array_equal(A.view, inputs.to16(A32, "bf16"))
    assert np.array_equal(B.view, inputs.to16(B32, "bf16"))
