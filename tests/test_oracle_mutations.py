"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them.

Each mutant is a textual edit of one oracle source compiled into a
temporary library; the pin battery runs in a subprocess (a mutant may read out
of bounds) and must report at least one failure or die.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gemm_oracle.c")
TRANSPOSE_SRC = os.path.join(ROOT, "oracle", "transpose_oracle.c")

MUTANTS = {
    "transposed_B_index": ("(double)B[k * b_rs + j * b_cs]", "(double)B[j * b_rs + k * b_cs]"),
    "A_uses_B_stride": ("(double)A[i * a_rs + k * a_cs]", "(double)A[i * b_rs + k * a_cs]"),
    "transpose_op_ignored": ("else         { *rs = 1;  *cs = ld; }", "else         { *rs = ld; *cs = 1; }"),
    "op_flags_swapped": ("op_strides(op_a, lda, &a_rs, &a_cs);\n    op_strides(op_b, ldb, &b_rs, &b_cs);\n\n    int64_t rows",
                         "op_strides(op_b, lda, &a_rs, &a_cs);\n    op_strides(op_a, ldb, &b_rs, &b_cs);\n\n    int64_t rows"),
    "entries_op_ignored": ("op_strides(op_a, lda, &a_rs, &a_cs);\n    op_strides(op_b, ldb, &b_rs, &b_cs);\n    for",
                           "op_strides(0, lda, &a_rs, &a_cs);\n    op_strides(0, ldb, &b_rs, &b_cs);\n    for"),
    "dropped_first_term": ("for (int64_t k = 0; k < K; ++k) {\n        double prod",
                           "for (int64_t k = 1; k < K; ++k) {\n        double prod"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double prod",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n        double prod"),
    "wrong_sign": ("acc += prod;", "acc -= prod;"),
    "single_precision_accumulator": ("double acc = 0.0;", "float acc = 0.0f;"),
    "magnitude_without_abs": ("mag += fabs(prod);", "mag += prod;"),
    "negative_zero_start": ("double acc = 0.0;", "double acc = -0.0;"),
    "swapped_output_index": ("job->C[i * job->ldc + j] = c;", "job->C[j * job->ldc + i] = c;"),
    "traffic_ghost_as_load": ("if (row < M && k < K) out[0]++; else out[2]++;",
                              "if (row <= M && k < K) out[0]++; else out[2]++;"),
    "traffic_B_tile_transposed": ("if (k < K && col < N) out[1]++; else out[3]++;",
                                  "if (k < N && col < K) out[1]++; else out[3]++;"),
    "bank_broadcast_counted": ("if (!seen)\n                distinct++;", "distinct++;"),
    # transpose_oracle.c
    "transpose_not_transposed": ("out[c * ld_out + r] = in[r * ld_in + c];",
                                 "out[r * ld_out + c] = in[r * ld_in + c];"),
    "transpose_wrong_in_ld": ("out[c * ld_out + r] = in[r * ld_in + c];",
                              "out[c * ld_out + r] = in[r * cols + c];"),
    "transpose_drops_last_row": ("for (int64_t r = 0; r < rows; ++r)\n        for (int64_t c = 0; c < cols; ++c)",
                                 "for (int64_t r = 0; r < rows - 1; ++r)\n        for (int64_t c = 0; c < cols; ++c)"),
    "sectors_end_byte_ignored": ("s <= (addr[l] + width - 1) / sector_bytes", "s <= addr[l] / sector_bytes"),
    "sectors_duplicates_counted": ("if (!dup)\n                seen[n++] = s;", "seen[n++] = s;"),
}
MUTANTS.update({
    # reduce_oracle.c
    "sum_skips_first": ("for (int64_t i = 0; i < n; ++i) {\n        s += (double)x[i];",
                        "for (int64_t i = 1; i < n; ++i) {\n        s += (double)x[i];"),
    "sum_single_precision": ("double s = 0.0, a = 0.0;", "float s = 0.0f; double a = 0.0;"),
    "sum_abs_missing": ("a += fabs((double)x[i]);", "a += (double)x[i];"),
    "tree_v0_condition": ("(tid % (2 * s) == 0)", "(tid % s == 0)"),
    "tree_counts_threads_not_warps": ("warps_here += any;", "warps_here += 1;"),
    "passes_floor_division": ("n = (n + per_block - 1) / per_block;", "n = n / per_block;"),
})
REDUCE_MUTANTS = {"sum_skips_first", "sum_single_precision", "sum_abs_missing", "tree_v0_condition",
                  "tree_counts_threads_not_warps", "passes_floor_division"}
REDUCE_SRC = os.path.join(ROOT, "oracle", "reduce_oracle.c")
MUTANTS.update({
    # gemm16_oracle.c
    "bf16_bias_off": ("v = ldexp(1.0 + f / 128.0, e - 127);", "v = ldexp(1.0 + f / 128.0, e - 126);"),
    "f16_subnormal_as_normal": ("v = ldexp((double)f, -24);", "v = ldexp(1.0 + f / 1024.0, -14);"),
    "f16_fraction_width": ("v = ldexp(1.0 + f / 1024.0, e - 15);", "v = ldexp(1.0 + f / 512.0, e - 15);"),
    "decode16_sign_ignored": ("return neg ? -v : v;", "return v;"),
    "gemm16_drops_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        const double prod",
                               "for (int64_t k = 0; k < K - 1; ++k) {\n        const double prod"),
    "gemm16_B_uses_lda": ("val[B[k * b_rs + j * b_cs]]", "val[B[k * a_rs + j * b_cs]]"),
    "gemm16_format_ignored": ("double *val = decode_table(format);\n    int64_t rows",
                              "double *val = decode_table(FMT_BF16);\n    int64_t rows"),
    "gemm16_transpose_ignored": ("    else         { *rs = 1;  *cs = ld; }\n}\n\n/* C (binary64",
                                 "    else         { *rs = ld; *cs = 1; }\n}\n\n/* C (binary64"),
    "gemm16_op_flags_swapped": ("op16_strides(op_a, lda, &a_rs, &a_cs);\n    op16_strides(op_b, ldb, &b_rs, &b_cs);\n    double *val = decode_table(format);\n    int64_t rows",
                                "op16_strides(op_b, lda, &a_rs, &a_cs);\n    op16_strides(op_a, ldb, &b_rs, &b_cs);\n    double *val = decode_table(format);\n    int64_t rows"),
    "gemm16_entries_op_ignored": ("op16_strides(op_a, lda, &a_rs, &a_cs);\n    op16_strides(op_b, ldb, &b_rs, &b_cs);\n    double *val = decode_table(format);\n    if (!val)",
                                  "op16_strides(0, lda, &a_rs, &a_cs);\n    op16_strides(0, ldb, &b_rs, &b_cs);\n    double *val = decode_table(format);\n    if (!val)"),
})
GEMM16_MUTANTS = {"bf16_bias_off", "f16_subnormal_as_normal", "f16_fraction_width", "decode16_sign_ignored",
                  "gemm16_drops_last_term", "gemm16_B_uses_lda", "gemm16_format_ignored",
                  "gemm16_transpose_ignored", "gemm16_op_flags_swapped", "gemm16_entries_op_ignored"}
GEMM16_SRC = os.path.join(ROOT, "oracle", "gemm16_oracle.c")
TRANSPOSE_MUTANTS = {"transpose_not_transposed", "transpose_wrong_in_ld", "transpose_drops_last_row",
                     "sectors_end_byte_ignored", "sectors_duplicates_counted"}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = TRANSPOSE_SRC if name in TRANSPOSE_MUTANTS else REDUCE_SRC if name in REDUCE_MUTANTS else \
        GEMM16_SRC if name in GEMM16_MUTANTS else SRC
    text = open(src).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(text.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(out=lib, replace={os.path.basename(src): str(mutant_src)})
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                          cwd=ROOT, capture_output=True, text=True, timeout=300,
                          env={**os.environ, "PYTHONPATH": ROOT})
    # exit 3: some pin failed; negative or other non-zero: the mutant crashed
    assert proc.returncode != 0, f"no pin caught mutant {name}: {proc.stdout}{proc.stderr}"
    if proc.returncode == 3:
        assert "FAILED:" in proc.stdout and proc.stdout.strip() != "FAILED:"
