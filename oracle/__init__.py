"""Float64 CPU oracle (test infrastructure only; see yoco_oracle)."""

from .yoco_oracle import (  # noqa: F401
    attention_one_query,
    cross_attention,
    cross_attention_varlen,
    cross_metadata,
    gather_rows,
    query_positions,
    dequantize_cache,
    e4m3_decode,
    e4m3_encode,
    gated_retention,
    kv_append_fp8,
    kv_scatter,
    quantize_rows,
    gather_last,
    kv_append,
    kv_project,
    logical_kv,
    rms_norm,
)
