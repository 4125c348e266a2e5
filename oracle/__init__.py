"""CPU oracle (float64) for paged and sparse MLA decode: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg use it.  It shares no code with the GPU library.
"""

from .mla_oracle import (  # noqa: F401
    E2M1_TABLE, E4M3_TABLE, attend, bf16_to_f64, e2m1_value, e4m3_encode, e4m3_value, fp4_rows_f64,
    fp8_cast_rows, fused_decode, gather_paged_fp4, gather_paged_records, gather_paged_rows, lse_combine,
    paged_decode, paged_decode_fp4, paged_decode_fp8, rms_norm, rope_rotate, round_bf16, sparse_decode,
    sparse_rows_f64, visible_count,
)
