"""MI355X-native batched speculative-decoding verification.

The verify path lives in ``libspecverify.so`` (HIP kernels for gfx950 behind
the C ABI in ``include/specverify.h``); ``specverify`` is its ctypes binding.
"""
from .specverify import (  # noqa: F401
    SV_BF16, SV_ESCRATCH, SV_F32, SV_NOALLOC_SCRATCH_BYTES, SpecVerifyError, Workspace, draft_window, kv_commit, kv_valid_slots, read_probe,
    row_softmax_stats, spec_read_probe, spec_read_probe_words,
    sample_rows, spec_draft_window, spec_draft_window_host, spec_draft_window_max_blocks, spec_kv_commit,
    spec_kv_valid_slots, spec_row_softmax_stats,
    spec_sample_rows, spec_sample_rows_workspace_bytes,
    spec_row_softmax_stats_workspace_bytes, spec_verify, spec_verify_ragged, spec_verify_ragged_workspace_bytes,
    spec_verify_noalloc, spec_verify_strerror, spec_verify_timing_enable, spec_verify_timing_read,
    spec_verify_timing_reset, spec_verify_tree,
    spec_verify_tree_lossless, spec_verify_tree_lossless_workspace_bytes,
    spec_verify_tree_workspace_bytes, spec_verify_version, spec_verify_workspace_bytes, verify_chain, verify_ragged,
    verify_tree, verify_tree_lossless,
)
