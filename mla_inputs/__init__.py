"""Seeded synthetic inputs for paged and sparse MLA decode.

This package only draws and lays out inputs: random numbers, block tables,
index lists, the bf16 rounding of drawn floats and the fp8 / fp4 quantisation of
the caches.  It computes nothing of the attention itself, so both the CPU
oracle and the GPU path can take their inputs from it.
"""

from .gen import (  # noqa: F401
    D_QK, D_V, PAGE, REC_BYTES,
    PagedInputs, PagedFp8Inputs, PagedFp4Inputs, SparseInputs,
    bf16_bits_from_f32, bf16_bits_to_f32, quantize_rows_nvfp4,
    make_paged, make_paged_fp8, make_paged_fp4, make_sparse, make_config, config_info, CONFIGS,
    FusedExtras, make_fused_extras, rope_angles,
)
