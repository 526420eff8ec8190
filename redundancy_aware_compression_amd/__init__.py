"""R-KV decode-time KV-cache eviction on AMD Instinct MI355X (gfx950).

The work happens in ``librkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rkv.h``). This module only marshals arguments to it with
ctypes; it has no compute of its own and no fallback: importing it fails
loudly when the library has not been built.

Pointers may be given as integers or as objects with ``data_ptr()`` (torch
tensors). ``stream`` defaults to torch's current HIP stream.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    RKV_BF16,
    RKV_F32,
    RKV_MAX_CAPACITY,
    RKV_MAX_LAYERS,
    RKV_MAX_QROWS,
    RKV_NOALLOC_WORKSPACE_BYTES,
    STATUS,
    RkvError,
    RkvParams,
    library_path,
    make_params,
    rkv_compact,
    rkv_compact_holefill,
    rkv_evict_step,
    rkv_evict_step_holefill,
    rkv_evict_step_holefill_timed,
    rkv_evict_step_sampled,
    rkv_evict_step_sentences,
    rkv_evict_step_captured,
    rkv_evict_step_noalloc,
    rkv_decode_attention,
    rkv_evict_step_timed,
    rkv_last_hip_error,
    rkv_score,
    rkv_select,
    rkv_select_sampled,
    rkv_sentence_penalty,
    rkv_status_string,
    rkv_workspace_bytes,
    rkv_workspace_keep_offset,
)
