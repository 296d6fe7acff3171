"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments synchronously with the documented codes."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f32.h")


def _header_text():
    text = open(HEADER).read()
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def declared_functions():
    """Every function the header declares (return type at the line start)."""
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int64_t|int|char|void)\s*\*?\s*(\w+)\s*\(",
                                 _header_text(), flags=re.M)))


def declared_codes():
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(GEMM_\w+)\s+(-?\d+)", _header_text())}


@pytest.fixture(scope="module")
def binding():
    from shared_memory_tiled_amd import binding as b
    b.load_library()
    return b


@pytest.fixture(scope="module")
def lib(binding):
    return binding.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"gemm_f32", "gemm_f32_variant", "gemm_f32_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gemm_f32.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "shared_memory_tiled_amd", "libgemm_f32.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT ([A-Za-z]\w*)$", out, flags=re.M))    # C names (no _Z, _init)
    assert exported == set(names), exported ^ set(names)
    assert {"transpose_f32", "reduce_sum_f32", "gemm_mixed", "gemm_mixed_variant"} <= set(names)


def test_library_is_independent_of_the_oracle():
    so = os.path.join(ROOT, "shared_memory_tiled_amd", "libgemm_f32.so")
    syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in syms
    needed = subprocess.run(["readelf", "-d", so], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in needed
    pkg = os.path.join(ROOT, "shared_memory_tiled_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "gemm_oracle" not in text, f


def test_status_codes_and_strings(binding):
    codes = declared_codes()
    statuses = {v for k, v in codes.items() if k.startswith(("GEMM_F32_OK", "GEMM_F32_ERR"))}
    assert statuses == set(range(len(statuses)))
    msgs = [binding.gemm_f32_status_string(s) for s in sorted(statuses)]
    assert msgs[0] == "ok" and len(set(msgs)) == len(msgs)
    assert binding.gemm_f32_status_string(999) == "unknown status"


def test_variant_names(binding):
    codes = declared_codes()
    n = binding.gemm_f32_num_variants()
    assert n == 4 and codes["GEMM_F32_VARIANT_MFMA"] == 3
    names = [binding.gemm_f32_variant_name(v) for v in range(n)]
    assert all(names) and len(set(names)) == n
    nd = binding.gemm_f32_num_diagnostic_variants()
    diag = [binding.gemm_f32_variant_name(16 + d) for d in range(nd)]
    assert all(diag) and len(set(diag)) == nd
    assert binding.gemm_f32_variant_name(n) is None
    assert binding.gemm_f32_variant_name(16 + nd) is None
    assert binding.gemm_f32_variant_name(-1) is None


FAKE = 0x10000          # an aligned, never dereferenced address


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((4, -2, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((4, 4, -3, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((4, 4, 8, FAKE, 7, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 6, 4, FAKE, 4, FAKE, 5, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 6, 4, FAKE, 4, FAKE, 6, FAKE, 5), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 4, 0, FAKE, 0, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 4, 4, None, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 4, 4, FAKE, 4, None, 4, FAKE, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 4, 4, FAKE, 4, FAKE, 4, None, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 4, 0, None, 1, None, 4, None, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 4, 4, FAKE + 2, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_MISALIGNED"),
    ((4, 4, 4, FAKE, 4, FAKE + 1, 4, FAKE, 4), "GEMM_F32_ERR_MISALIGNED"),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE + 3, 4), "GEMM_F32_ERR_MISALIGNED"),
    ((2**31, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_TOO_LARGE"),
    ((4, 4, 2**31, FAKE, 2**31, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_TOO_LARGE"),
    ((4, 4, 4, FAKE, 2**62, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_TOO_LARGE"),
    ((2**30, 2**30, 4, FAKE, 4, FAKE, 2**30, FAKE, 2**30), "GEMM_F32_ERR_TOO_LARGE"),
    ((0, 4, 4, None, 4, None, 4, None, 4), "GEMM_F32_OK"),      # empty: no launch
    ((4, 0, 4, None, 4, None, 1, None, 1), "GEMM_F32_OK"),
])
def test_validation_without_launch(lib, args, code):
    want = declared_codes()[code]
    M, N, K, A, lda, B, ldb, C, ldc = args
    assert lib.gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, None) == want
    for v in (0, 1, 2, 3, 16):
        assert lib.gemm_f32_variant(v, M, N, K, A, lda, B, ldb, C, ldc, None) == want


@pytest.mark.parametrize("op_a,op_b,args,code", [
    (2, 0, (4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_OP"),
    (0, -1, (4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_OP"),
    (1, 0, (8, 4, 3, FAKE, 7, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),    # A^T: lda >= M
    (1, 0, (8, 4, 3, FAKE, 8, FAKE, 4, FAKE, 4), "GEMM_F32_OK_IF_NO_GPU"),
    (0, 1, (4, 6, 9, FAKE, 9, FAKE, 8, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),    # B^T: ldb >= K
    (1, 1, (4, 6, 9, FAKE, 3, FAKE, 9, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),
    (1, 1, (4, 6, 9, FAKE + 1, 4, FAKE, 9, FAKE, 6), "GEMM_F32_ERR_MISALIGNED"),
    (1, 0, (-1, 6, 9, FAKE, 4, FAKE, 6, FAKE, 6), "GEMM_F32_ERR_INVALID_DIM"),
    (1, 1, (0, 6, 9, None, 1, None, 9, None, 6), "GEMM_F32_OK"),
])
def test_op_validation_without_launch(lib, op_a, op_b, args, code):
    if code == "GEMM_F32_OK_IF_NO_GPU":
        return      # valid arguments: would launch (covered by the GPU tests)
    want = declared_codes()[code]
    assert lib.gemm_f32_op(op_a, op_b, *args, None) == want


def test_unknown_variant(lib):
    code = declared_codes()["GEMM_F32_ERR_INVALID_VARIANT"]
    for v in (4, 15, -1, 16 + lib.gemm_f32_num_diagnostic_variants(), 1000):
        assert lib.gemm_f32_variant(v, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None) == code


def test_python_errors_are_raised(binding):
    with pytest.raises(binding.GemmError) as e:
        binding.gemm_f32(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, stream=0)
    assert e.value.status == declared_codes()["GEMM_F32_ERR_INVALID_DIM"]


@pytest.mark.parametrize("args,code", [
    ((-1, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((4, -1, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((4, 6, FAKE, 5, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 6, FAKE, 6, FAKE, 3), "GEMM_F32_ERR_INVALID_LD"),
    ((4, 6, None, 6, FAKE, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 6, FAKE, 6, None, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 6, FAKE + 2, 6, FAKE, 4), "GEMM_F32_ERR_MISALIGNED"),
    ((2**31, 6, FAKE, 6, FAKE, 2**31), "GEMM_F32_ERR_TOO_LARGE"),
    ((0, 6, None, 6, None, 1), "GEMM_F32_OK"),
    ((6, 0, None, 1, None, 6), "GEMM_F32_OK"),
])
def test_transpose_validation_without_launch(lib, args, code):
    want = declared_codes()[code]
    assert lib.transpose_f32(*args, None) == want
    for v in range(lib.transpose_f32_num_variants()):
        assert lib.transpose_f32_variant(v, *args, None) == want


def test_transpose_variants(binding, lib):
    n = binding.transpose_f32_num_variants()
    names = [binding.transpose_f32_variant_name(v) for v in range(n)]
    assert n == 11 and all(names) and len(set(names)) == n
    assert binding.transpose_f32_variant_name(n) is None
    code = declared_codes()["GEMM_F32_ERR_INVALID_VARIANT"]
    assert lib.transpose_f32_variant(n, 4, 4, FAKE, 4, FAKE, 4, None) == code


@pytest.mark.parametrize("args,code", [
    ((-1, FAKE, FAKE, FAKE, 4096), "GEMM_F32_ERR_INVALID_DIM"),
    ((10, FAKE, None, FAKE, 4096), "GEMM_F32_ERR_NULL_PTR"),
    ((10, None, FAKE, FAKE, 4096), "GEMM_F32_ERR_NULL_PTR"),
    ((10, FAKE + 2, FAKE, FAKE, 4096), "GEMM_F32_ERR_MISALIGNED"),
    ((10**6, FAKE, FAKE, FAKE, 4), "GEMM_F32_ERR_WORKSPACE"),
    ((10**6, FAKE, FAKE, None, 10**8), "GEMM_F32_ERR_NULL_PTR"),
    ((2**40, FAKE, FAKE, FAKE, 2**45), "GEMM_F32_ERR_TOO_LARGE"),
])
def test_reduce_validation_without_launch(lib, args, code):
    want = declared_codes()[code]
    n, x, out, ws, wsb = args
    for v in (0, 1, 2, 4):
        assert lib.reduce_sum_f32_variant(v, n, x, out, ws, wsb, None) == want, v


@pytest.mark.parametrize("args,code", [
    ((0, -1, FAKE, FAKE), "GEMM_F32_ERR_INVALID_DIM"),
    ((7, 10, FAKE, FAKE), "GEMM_F32_ERR_INVALID_VARIANT"),
    ((-1, 10, FAKE, FAKE), "GEMM_F32_ERR_INVALID_VARIANT"),
    ((1, 10, FAKE, None), "GEMM_F32_ERR_NULL_PTR"),
    ((2, 10, None, FAKE), "GEMM_F32_ERR_NULL_PTR"),
    ((4, 10, FAKE + 2, FAKE), "GEMM_F32_ERR_MISALIGNED"),
    ((4, 2**40, FAKE, FAKE), "GEMM_F32_ERR_TOO_LARGE"),
    # versions 0-2 keep ~n/255 partials: past 1 MiB of them the fixed scratch
    # is too small, and the call is refused before anything is enqueued
    ((0, 2**27, FAKE, FAKE), "GEMM_F32_ERR_SCRATCH"),
    ((1, 2**27, FAKE, FAKE), "GEMM_F32_ERR_SCRATCH"),
    ((2, 10**9, FAKE, FAKE), "GEMM_F32_ERR_SCRATCH"),
])
def test_reduce_noalloc_validation_without_launch(lib, args, code):
    assert lib.reduce_sum_f32_variant_noalloc(*args, None) == declared_codes()[code]


@pytest.mark.parametrize("args,code", [
    ((4, FAKE, 1, FAKE), "GEMM_F32_ERR_INVALID_VARIANT"),
    ((-1, FAKE, 1, FAKE), "GEMM_F32_ERR_INVALID_VARIANT"),
    ((2, FAKE, -1, FAKE), "GEMM_F32_ERR_INVALID_DIM"),
    ((2, None, 1, FAKE), "GEMM_F32_ERR_NULL_PTR"),
    ((2, FAKE, 1, None), "GEMM_F32_ERR_NULL_PTR"),
    ((2, FAKE + 2, 1, FAKE), "GEMM_F32_ERR_MISALIGNED"),
])
def test_lds_probe_validation_without_launch(lib, args, code):
    assert lib.gemm_f32_lds_probe(*args, None) == declared_codes()[code]


@pytest.mark.parametrize("args,code", [
    ((2, 1, 2, FAKE, FAKE, FAKE), "GEMM_F32_ERR_INVALID_VARIANT"),
    ((0, 0, 2, FAKE, FAKE, FAKE), "GEMM_F32_ERR_INVALID_DIM"),
    ((0, 1, 3, FAKE, FAKE, FAKE), "GEMM_F32_ERR_INVALID_DIM"),
    ((1, 1, -2, FAKE, FAKE, FAKE), "GEMM_F32_ERR_INVALID_DIM"),
    ((0, 1, 2, None, FAKE, FAKE), "GEMM_F32_ERR_NULL_PTR"),
    ((0, 1, 2, FAKE, FAKE, None), "GEMM_F32_ERR_NULL_PTR"),
    ((0, 1, 2, FAKE + 4, FAKE, FAKE), "GEMM_F32_ERR_MISALIGNED"),
    ((0, 1, 2, FAKE, FAKE, FAKE + 4), "GEMM_F32_ERR_MISALIGNED"),
    ((0, 2**31, 2, FAKE, FAKE, FAKE), "GEMM_F32_ERR_TOO_LARGE"),
])
def test_copy_probe_validation_without_launch(lib, args, code):
    assert lib.gemm_f32_copy_probe(*args, None) == declared_codes()[code]


@pytest.mark.parametrize("args,code", [
    ((64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 16), "GEMM_F32_ERR_INVALID_DIM"),
    ((64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 48), "GEMM_F32_ERR_INVALID_DIM"),
    ((64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, None, 64), "GEMM_F32_ERR_NULL_PTR"),
    ((64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE + 2, 64), "GEMM_F32_ERR_MISALIGNED"),
    ((64, 64, 6, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64), "GEMM_F32_ERR_INVALID_DIM"),   # K % 4 != 0
    ((0, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64), "GEMM_F32_ERR_INVALID_DIM"),
    ((64, 64, 64, FAKE, 32, FAKE, 64, FAKE, 64, FAKE, 64), "GEMM_F32_ERR_INVALID_LD"),
    ((64, 64, 64, None, 64, FAKE, 64, FAKE, 64, FAKE, 64), "GEMM_F32_ERR_NULL_PTR"),
])
def test_ksplit_timeline_validation_without_launch(lib, args, code):
    assert lib.gemm_f32_ksplit_timeline(*args, None) == declared_codes()[code]


def test_reduce_noalloc_scratch_limit(binding):
    """The declared scratch size, and the largest n each tree version takes
    in it: exactly where the workspace the version needs passes 1 MiB."""
    text = open(HEADER).read()
    assert re.search(r"#define\s+REDUCE_SUM_F32_SCRATCH_BYTES\s+\(1 << 20\)", text)
    limit = binding.REDUCE_SCRATCH_BYTES
    assert limit == 1 << 20
    for v in (0, 1, 2):
        lo, hi = 1, 2**30          # largest n whose workspace fits in the scratch
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if binding.reduce_sum_f32_workspace_size(v, mid) <= limit:
                lo = mid
            else:
                hi = mid - 1
        assert 6.6e7 < lo < 6.8e7, lo
    for v in (3, 4):
        assert binding.reduce_sum_f32_workspace_size(v, 2**39) <= limit


def test_reduce_workspace_sizes(binding, lib):
    # the page's multi-pass sizes: 2^24 values -> 65,536 + 256 partials kept
    assert binding.reduce_sum_f32_workspace_size(1, 2**24) == 4 * (65536 + 256)
    assert binding.reduce_sum_f32_workspace_size(0, 256) == 0
    assert binding.reduce_sum_f32_workspace_size(2, 257) == 4 * 2
    assert binding.reduce_sum_f32_workspace_size(3, 10**9) == 0
    assert binding.reduce_sum_f32_workspace_size(4, 1) == 4 * 2048


@pytest.mark.parametrize("args,code", [
    ((2, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_FORMAT"),
    ((-1, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_FORMAT"),
    ((0, -1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((1, 4, 4, -3, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_DIM"),
    ((0, 4, 4, 8, FAKE, 7, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),
    ((1, 4, 6, 4, FAKE, 4, FAKE, 5, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),
    ((0, 4, 6, 4, FAKE, 4, FAKE, 6, FAKE, 5), "GEMM_F32_ERR_INVALID_LD"),
    ((0, 4, 4, 4, None, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((1, 4, 4, 4, FAKE, 4, None, 4, FAKE, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((0, 4, 4, 4, FAKE, 4, FAKE, 4, None, 4), "GEMM_F32_ERR_NULL_PTR"),
    ((0, 4, 4, 4, FAKE + 1, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_MISALIGNED"),   # 16-bit: 2-byte alignment
    ((1, 4, 4, 4, FAKE, 4, FAKE + 3, 4, FAKE, 4), "GEMM_F32_ERR_MISALIGNED"),
    ((0, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE + 2, 4), "GEMM_F32_ERR_MISALIGNED"),   # C is binary32
    ((0, 2**31, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_TOO_LARGE"),
    ((1, 4, 4, 4, FAKE, 2**62, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_TOO_LARGE"),
    ((0, 0, 4, 4, None, 4, None, 4, None, 4), "GEMM_F32_OK"),          # empty: no launch
    ((1, 4, 0, 4, None, 4, None, 1, None, 1), "GEMM_F32_OK"),
])
def test_mixed_validation_without_launch(lib, args, code):
    want = declared_codes()[code]
    assert lib.gemm_mixed(*args, None) == want
    for v in range(lib.gemm_mixed_num_variants()):
        assert lib.gemm_mixed_variant(v, *args, None) == want


def test_mixed_variants(binding, lib):
    n = binding.gemm_mixed_num_variants()
    names = [binding.gemm_mixed_variant_name(v) for v in range(n)]
    assert n >= 3 and all(names) and len(set(names)) == n
    assert binding.gemm_mixed_variant_name(n) is None and binding.gemm_mixed_variant_name(-1) is None
    code = declared_codes()["GEMM_F32_ERR_INVALID_VARIANT"]
    assert lib.gemm_mixed_variant(n, 0, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, None) == code
    assert declared_codes()["GEMM_MIXED_BF16"] == binding.FORMATS["bf16"] == 0
    assert declared_codes()["GEMM_MIXED_F16"] == binding.FORMATS["f16"] == 1
    assert binding.reduce_sum_f32_workspace_size(9, 10) == -1
    assert binding.reduce_sum_f32_workspace_size(1, -1) == -1
    n = binding.reduce_sum_f32_num_variants()
    names = [binding.reduce_sum_f32_variant_name(v) for v in range(n)]
    assert n == 5 and all(names) and len(set(names)) == n and binding.reduce_sum_f32_variant_name(n) is None


@pytest.mark.parametrize("op_a,op_b,args,code", [
    (2, 0, (0, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_OP"),
    (0, -1, (0, 4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_OP"),
    (1, 0, (0, 8, 4, 3, FAKE, 7, FAKE, 4, FAKE, 4), "GEMM_F32_ERR_INVALID_LD"),     # A^T: lda >= M
    (0, 1, (1, 4, 6, 9, FAKE, 9, FAKE, 8, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),     # B^T: ldb >= K
    (1, 1, (0, 4, 6, 9, FAKE, 3, FAKE, 9, FAKE, 6), "GEMM_F32_ERR_INVALID_LD"),
    (1, 1, (5, 4, 6, 9, FAKE, 4, FAKE, 9, FAKE, 6), "GEMM_F32_ERR_INVALID_FORMAT"),
    (1, 1, (0, 4, 6, 9, FAKE + 1, 4, FAKE, 9, FAKE, 6), "GEMM_F32_ERR_MISALIGNED"),
    (1, 0, (1, -1, 6, 9, FAKE, 4, FAKE, 6, FAKE, 6), "GEMM_F32_ERR_INVALID_DIM"),
    (1, 1, (0, 0, 6, 9, None, 1, None, 9, None, 6), "GEMM_F32_OK"),
])
def test_mixed_op_validation_without_launch(lib, op_a, op_b, args, code):
    assert lib.gemm_mixed_op(op_a, op_b, *args, None) == declared_codes()[code]


def test_default_variant_choices(binding):
    """The configuration the default entry points run, by problem size (no
    device needed).  Shapes the four-wave schedule takes (K, M and N
    multiples of 4): its 256 x 256 tiles when at least 256 of them fill their
    rounds of 256 to 95 %, else its 128 x 128 tiles when there are at least
    128, else the split-phase 64 x 64 tiles.  Other shapes: eight-wave 256 x
    256 tiles when their rounds run at least 80 % full (75 % when 128 x 128
    tiles would not fill theirs to 90 %), register-staged 128 x 128 tiles
    when at least 256 of them fill their rounds to 90 %, else the split-phase
    tiles (32-deep phases for at most 256 tiles).  Then, with K, M and N
    multiples of 4, the 64 x 64 tiles whose four waves split the phases where
    a cost model of rounds, efficiency and fixed cost per tile gives them the
    shorter time (K >= 448), or in place of the split-phase tiles (K >= 384),
    and the 96 x 96 ones where the same model gives those the shorter time.
    Last, at most 512 output tiles of 16 x 16 take the 16 x 16 small-tile
    kernel on 8 waves, at most 1024 the 32 x 32 one on 4 waves, whatever K.
    For the 16-bit product the
    scheduled kernel from 128 tiles of 256 x 256, else the k-split 64 x 64
    tiles below 128 tiles of 128 x 128 (K a multiple of 8), else 128 x 128
    direct copies from 128 tiles of those (64 for K >= 2048), else 64 x 64
    tiles.  Invalid sizes give -1."""
    f32 = {
        (8192, 8192, 8192): "mfma256x256_bk32_w2x2_sched",
        (4096, 4096, 4096): "mfma256x256_bk32_w2x2_sched",
        (8192, 4096, 2048): "mfma256x256_bk32_w2x2_sched",
        (4096, 4096, 32): "mfma256x256_bk32_w2x2_sched",
        (7940, 8132, 32): "mfma256x256_bk32_w2x2_sched",         # 1024 tiles with edges
        (8200, 8200, 8192): "mfma96x96_bk16_w1x1_k4_sched",       # 1089 tiles of 256: 85 % of 5 rounds
        (4100, 4104, 4096): "mfma64x64_bk32_w1x1_k4_sched",       # 4225 tiles of 64: 16.5 rounds
        (4000, 5000, 4096): "mfma128x128_bk32_w2x2_sched",
        (2048, 2048, 2048): "mfma128x128_bk32_w2x2_sched",
        (6144, 6144, 6144): "mfma128x128_bk32_w2x2_sched",
        (7168, 7168, 7168): "mfma96x96_bk16_w1x1_k4_sched",       # 5625 tiles of 96: 21.97 rounds
        (3000, 3000, 384): "mfma64x64_bk32_w2x2_sched",          # 2209 tiles of 64, four per CU
        (2048, 3072, 512): "mfma64x64_bk32_w2x2_sched",
        (3072, 3072, 768): "mfma64x64_bk32_w2x2_sched",
        (3000, 7000, 1024): "mfma64x64_bk32_w2x2_sched",
        (2048, 2048, 256): "mfma128x128_bk32_w2x2_sched",        # 256 tiles of 128: one round
        (2048, 2048, 512): "mfma128x128_bk32_w2x2_sched",
        (4096, 4096, 256): "mfma256x256_bk32_w2x2_sched",
        (1024, 1024, 512): "mfma64x64_bk32_w1x1_k4_sched",
        (3072, 3072, 3072): "mfma96x96_bk16_w1x1_k4_sched",       # 1024 tiles of 96: 4 full rounds
        (1536, 1536, 1536): "mfma96x96_bk16_w1x1_k4_sched",       # 256 tiles of 96: one round
        (5120, 5120, 5120): "mfma64x64_bk32_w1x1_k4_sched",       # 6400 tiles of 64: 25 full rounds
        (1024, 1024, 1024): "mfma64x64_bk32_w1x1_k4_sched",
        (4096, 4096, 48): "mfma256x256_bk32_w2x2_sched",          # K % 32 = 16: last phase past K
        (8193, 8190, 96): "mfma256x256_bk32_w2x4_direct",
        (4096, 4096, 0): "mfma256x256_bk32_w2x4_direct",
        (6000, 6000, 6000): "mfma128x128_bk32_w2x2_sched",        # K % 32 = 16: last phase past K
        (5000, 3000, 2000): "mfma128x128_bk32_w2x2_sched",
        (4608, 4608, 4608): "mfma96x96_bk16_w1x1_k4_sched",       # 2304 tiles of 96: 9 full rounds
        (3840, 2048, 100): "mfma128x128_bk32_w2x2_sched",
        (3840, 2048, 102): "mfma128x128_bk16_w2x2",               # K % 4 = 2
        (4100, 4097, 515): "mfma64x64_bk16_w2x2_k4",              # K % 4 = 3
        (3000, 3000, 3000): "mfma96x96_bk16_w1x1_k4_sched",       # 1024 tiles of 96
        (2300, 2300, 2304): "mfma64x64_bk32_w1x1_k4_sched",
        (1000, 1000, 1000): "mfma64x64_bk32_w1x1_k4_sched",
        (1000, 2000, 500): "mfma64x64_bk32_w2x2_sched",          # 512 tiles of 64, two per CU
        (1000, 1000, 380): "mfma64x64_bk32_w2x2_k4",              # K < 384
        (1002, 1000, 1000): "mfma64x64_bk32_w2x2_k4",             # M % 4 = 2
        (256, 256, 256): "mfma16x16_w8_small",                   # 256 tiles of 16 x 16
        (1, 1, 1): "mfma16x16_w8_small",
        (256, 256, 0): "mfma16x16_w8_small",
        (128, 128, 8192): "mfma16x16_w8_small",
        (368, 352, 97): "mfma16x16_w8_small",                     # 506 tiles, ragged K
        (512, 512, 512): "mfma32x32_w4_small",                    # 1024 tiles of 16 x 16
        (4096, 64, 256): "mfma32x32_w4_small",
        (500, 400, 257): "mfma32x32_w4_small",
        (640, 640, 640): "mfma64x64_bk32_w1x1_k4_sched",          # 1600 tiles of 16 x 16
        (528, 512, 512): "mfma64x64_bk32_w1x1_k4_sched",          # 1056
        (1000, 1000, 380): "mfma64x64_bk32_w2x2_k4",
    }
    for (M, N, K), name in f32.items():
        v = binding.gemm_f32_default_variant(M, N, K)
        assert binding.gemm_f32_variant_name(v) == name, (M, N, K, v)
    mixed = {
        (8192, 8192, 8192): "mixed256x256_bk64_w4_wide",
        (4096, 4096, 64): "mixed256x256_bk64_w4_wide",
        (3072, 3072, 3072): "mixed192x192_bk64_w4_wide",          # one round of 256 tiles of 192
        (3072, 3072, 3071): "mixed256x256_bk64_w4_wide",          # odd K
        (4100, 4100, 4096): "mixed192x192_bk64_w4_wide",          # 2 rounds of 192 (484) as of 256 (289)
        (3584, 3584, 3584): "mixed256x256_bk64_w4_wide",          # 196 tiles of 256, 361 of 192
        (4608, 4608, 4608): "mixed256x256_rowsplit",              # 324 tiles of 256: last round 68
        (4352, 4352, 4352): "mixed256x256_rowsplit",              # 289: last round 33
        (4352, 4352, 4350): "mixed256x256_bk64_w4_wide",          # K % 8 != 0
        (7168, 7168, 7168): "mixed256x256_rowsplit",              # 784: last round 16
        (5120, 5120, 5120): "mixed256x256_bk64_w4_wide",          # 400: last round 144
        (8192, 4096, 2048): "mixed256x256_bk64_w4_wide",          # 512: two full rounds
        (2048, 4096, 1024): "mixed192x192_bk64_w4_wide",          # 128 tiles of 256, 242 of 192
        (1024, 8192, 2048): "mixed256x256_bk64_w4_wide",          # 258 tiles of 192: 2 rounds
        (2816, 2816, 2816): "mixed192x192_bk64_w4_wide",          # 121 of 256, 225 of 192
        (2816, 2816, 1024): "mixed192x192_bk64_w4_wide",          # 324 tiles of 160: 2 rounds
        (2560, 2560, 2560): "mixed160x160_bk64_w4_wide",          # 196 of 192, 256 of 160: 1 round
        (2304, 2304, 2304): "mixed160x160_bk64_w4_wide",          # 144 tiles of 192, 225 of 160
        (1280, 5120, 2048): "mixed160x160_bk64_w4_wide",          # 189 of 192, 256 of 160
        (2390, 2470, 200): "mixed160x160_bk64_w4_wide",           # 169 of 192, 240 of 160
        (1024, 4096, 1024): "mixed128x128_bk32_w4_ksplit",        # 256 tiles of 128, long K
        (1536, 2560, 768): "mixed128x128_bk64_w2x2_directAB",     # 112 tiles of 192
        (2560, 2560, 2561): "mixed128x128_bk64_w2x2_directAB",    # odd K
        (2048, 2048, 2048): "mixed128x128_bk32_w4_ksplit",        # 256 tiles of 128, long K
        (1536, 1536, 1536): "mixed128x128_bk32_w4_ksplit",        # 144 tiles of 128
        (2048, 2048, 256): "mixed128x128_bk64_w2x2_directAB",     # 256 tiles of 128, short K
        (2048, 2048, 2044): "mixed128x128_bk64_w2x2_directAB",    # K % 8 = 4, 256 tiles of 128, long K
        (1024, 1024, 4096): "mixed64x64_bk32_w4_ksplit",          # 64 tiles of 128: k-split
        (1024, 1024, 1024): "mixed64x64_bk32_w4_ksplit",
        (1000, 1000, 1000): "mixed64x64_bk32_w4_ksplit",
        (512, 512, 8192): "mixed64x64_bk32_w4_ksplit",
        (1024, 1024, 4092): "mixed128x128_bk64_w2x2_directAB",    # K % 8 = 4, long K: 64 tiles of 128
        (1000, 1000, 2002): "mixed160x160_bk64_w4_wide",          # K % 4 = 2, 64 tiles of 128
        (800, 1200, 3002): "mixed160x160_bk64_w4_wide",           # K % 4 = 2, 35 tiles of 192
        (1000, 2000, 500): "mixed160x160_bk64_w4_wide",           # K % 8 = 4: 66 tiles of 192
        (1536, 1536, 1538): "mixed128x128_bk64_w2x2_directAB",    # K % 8 = 2, 144 tiles of 128, long K
        (512, 512, 1002): "mixed64x64_bk64_w1x2",                 # K % 8 = 2, 9 tiles of 192
        (1000, 1000, 1001): "mixed64x64_bk64_w1x2",
    }
    for (M, N, K), name in mixed.items():
        assert binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K)) == name, (M, N, K)
    for bad in ((-1, 5, 5), (5, -1, 5), (5, 5, -1), (1 << 31, 5, 5)):
        assert binding.gemm_f32_default_variant(*bad) == -1
        assert binding.gemm_mixed_default_variant(*bad) == -1


def test_transpose_default_variant(binding):
    """transpose_f32's choice: nontemporal stores (9) for a square 64 x 64 tile
    grid or an input of 128 MiB or more, else cached stores (6)."""
    name = lambda r, c, li, lo: binding.transpose_f32_variant_name(binding.transpose_f32_default_variant(r, c, li, lo))
    assert name(8192, 8192, 8192, 8192) == "tile64_vec_diag_ntstore"
    assert name(4096, 4096, 4096, 4096) == "tile64_vec_diag_ntstore"
    assert name(12000, 6000, 6000, 12000) == "tile64_vec_diag_ntstore"
    assert name(8192, 2048, 2056, 8192) == "tile64_vec_diag"
    assert name(300, 200, 200, 300) == "tile64_vec_diag"
    assert binding.transpose_f32_default_variant(-1, 5, 5, 5) == -1
