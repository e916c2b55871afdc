"""MI355X-native TriAttention KV-cache pruning: Python face of libtriattn.so.

The hot path (score, top-B select, compaction) and the calibration run as
HIP kernels for gfx950 behind the C ABI in include/triattn.h; this package
only marshals arguments to it.  Importing raises if the library is not built.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, Decode, TriError, TriKvPages, TriShape, last_error, make_pages,
    make_shape, status_string, TRI_REDUCE_MAX, TRI_REDUCE_MEAN, TRI_ROPE_HALF_SPLIT,
    TRI_ROPE_INTERLEAVED, TRI_SCORE_WAIT_GAVE_UP, tri_calibrate, tri_calibrate_workspace_bytes,
    tri_debug_set_resident_groups, tri_debug_set_wait_limit, tri_debug_set_phase_buffer,
    PHASE_NAMES,
    tri_pyramid_budgets,
    tri_score, tri_score_noalloc, tri_score_offsets, tri_score_paged, tri_score_status,
    tri_select_compact,
    tri_select_compact_layers,
    tri_select_compact_paged, tri_stream_probe, tri_trig_correlation,
    tri_trig_correlation_workspace_bytes,
    tri_workspace_bytes, tri_workspace_bytes_layers, tri_workspace_bytes_offsets,
    tri_workspace_bytes_paged,
)
