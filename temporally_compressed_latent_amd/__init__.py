"""MI355X-native MTLA hot path: merge/append into a temporally compressed
latent cache, absorbed-form decode, stride-masked parallel prefill, the
decoder layer around them, and the training backward of the parallel pass.

The compute runs in libmtla.so (hand-written HIP kernels for gfx950 behind a
C ABI, declared in include/mtla.h).  This package is its thin binding; torch
is used only for device memory and streams.
"""
from ._lib import (  # noqa: F401
    LIB_PATH, MTLA_BF16, MTLA_ERR_HIP, MTLA_ERR_INVALID_ARG, MTLA_ERR_UNSUPPORTED,
    MTLA_ERR_WORKSPACE, MTLA_FLAG_GATE_PER_POSITION, MTLA_FLAG_PORTABLE, MTLA_FP32, MTLA_OK, MtlaDims, MtlaError,
    decode_attention_workspace, header_symbols, last_error, lib, make_dims, mtla_absorb_query,
    mtla_debug_slot_limits, mtla_debug_stride_mask, mtla_decode, mtla_decode_attention,
    mtla_decode_attention_workspace_bytes, mtla_decode_plan, mtla_decode_step, mtla_decode_step_noalloc,
    mtla_decode_workspace_bytes, mtla_merge_append,
    mtla_prefill, mtla_prefill_at, mtla_prefill_at_workspace_bytes, mtla_prefill_workspace_bytes,
    mtla_reorder_state, mtla_sinusoidal_pe, mtla_up_project, mtla_project_inputs, mtla_output_project,
    mtla_layer_decode_workspace_bytes, mtla_layer_decode_step, mtla_layer_prefill_workspace_bytes,
    mtla_layer_prefill, mtla_prefill_backward, mtla_prefill_backward_workspace_bytes,
    mtla_version, status_string, mtla_calib_stream_read, mtla_calib_mfma, mtla_calib_empty, mtla_calib_tile_stream,
    mtla_calib_load_pattern, mtla_calib_step_timeline, mtla_w_uv_tiles_bytes, mtla_pack_w_uv_tiles, mtla_decode_step_tiles,
    mtla_layer_decode_step_tiles,
    mtla_prefill_partials, mtla_prefill_keys, mtla_prefill_attention, prefill_slot_keys,
)
