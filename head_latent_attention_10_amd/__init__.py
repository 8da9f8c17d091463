"""MLA decode over a paged latent KV cache, hand-written HIP for MI355X (gfx950).

The compute lives in libmla_hip.so (C ABI, include/mla.h); this package is a
thin ctypes binding (`_lib`) plus device-memory plumbing (`device`).
"""
from ._lib import (  # noqa: F401
    MLA_BF16, MLA_F32, MLA_FP8_E4M3, MlaDecodeParams, MlaError, load_library, make_params,
    mla_absorb_q, mla_absorbed_dtype, mla_attend_latent, mla_attend_partial, mla_combine, mla_decode, mla_decode_num_splits,
    mla_decode_workspace_size, mla_gather_cache, mla_last_error, mla_partials_layout, mla_split_begin,
    mla_split_owner, mla_split_plan, mla_status_string, mla_up_project)
