"""Sparse-MQA decode path for AMD MI355X (gfx950): FP8 indexer scoring, top-k
selection and attention over FP4 latent rows plus an FP8 sliding window.

The computation lives in libsmqa.so (HIP kernels behind the C ABI declared in
include/smqa.h); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    Batch, Layout, SmqaError, load, version, sparse_mqa_score, sparse_mqa_score_fp8mma, topk_select,
    sparse_mqa_attend,
    sparse_mqa_attend_fp8kv, sparse_mqa_attend_nvfp4, sparse_mqa_attend_fused, sparse_mqa_attend_mxfp8q,
    decode_step, decode_step_fused, decode_step_noalloc, decode_step_workspace_size, LIB_PATH,
    DEBUG_LIB_PATH, debug_build, debug_flags, SMQA_DEBUG_POSITION, SMQA_DEBUG_E8M0, SMQA_DEBUG_LAYOUT,
    SMQA_DEBUG_CAND,
)
