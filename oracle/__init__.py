"""fp64 CPU oracle of the DeltaKV hot path (test infrastructure only; see
deltakv_oracle for the statement of what it computes)."""
from .deltakv_oracle import *  # noqa: F401,F403
from .deltakv_oracle import (  # noqa: F401
    rnd, n_refs, ref_positions, nonref_positions, idx_bytes_for, stream_bytes,
    cache_array_bytes, cache_bytes, dense_kv_bytes, decode_effective_bytes,
    shared_component, center, cosines, search, encode, compress_stream, compress, append_token,
    reconstruct_stream, attend, decode, decode_selected, quantize_q4, dequantize_q4, encode_exact,
    search_topk, mean_refs, ref_count, ref_rows, group_order, group_cache,
    ELEM_BYTES, ALIGN,
)
