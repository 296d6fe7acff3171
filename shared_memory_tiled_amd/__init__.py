"""MI355X (gfx950) fp32 GEMM built on shared-memory (LDS) tiling.

The compute path is the C-ABI library ``libgemm_f32.so`` (hand-written HIP
kernels for CDNA4); ``shared_memory_tiled_amd.binding`` marshals arguments to
it.  The binding is imported lazily so that ``shared_memory_tiled_amd.inputs``
can be used without loading torch or the GPU library.
"""
from __future__ import annotations

_BINDING_NAMES = {
    "gemm_f32", "gemm_f32_variant", "gemm_f32_num_variants",
    "gemm_f32_variant_name", "gemm_f32_status_string", "gemm", "GemmError",
    "gemm_f32_num_diagnostic_variants", "DIAGNOSTIC_BASE", "gemm_f32_op", "OPS",
    "transpose_f32", "transpose_f32_variant", "transpose_f32_num_variants",
    "transpose_f32_variant_name", "transpose",
    "reduce_sum_f32", "reduce_sum_f32_variant", "reduce_sum_f32_num_variants",
    "reduce_sum_f32_variant_name", "reduce_sum_f32_workspace_size", "reduce_sum",
    "gemm_mixed", "gemm_mixed_variant", "gemm_mixed_op", "gemm_mixed_num_variants", "gemm_mixed_variant_name",
    "gemm_f32_default_variant", "gemm_mixed_default_variant", "transpose_f32_default_variant",
    "gemm16", "FORMATS",
    "VARIANTS", "load_library", "library_path",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
