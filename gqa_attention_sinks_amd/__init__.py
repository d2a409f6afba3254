"""Grouped-query flash attention with per-head learned sinks for MI355X (gfx950).

The compute lives in ``libsinkattn.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/sinkattn.h``).  This package is the thin Python
binding (``binding``) plus the seeded input generators (``workloads``).
Importing it does not load the library; the first call does, and raises
``SinkAttnError`` if the library has not been built.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    SinkAttnError,
    abi_version,
    append_paged_kv_rope,
    balanced_segments,
    balanced_workspace_segments,
    balanced_workspace_views,
    decode_balanced_workspace_bytes,
    decode_paged,
    decode_paged_balanced,
    decode_paged_multi,
    decode_paged_noalloc,
    kv_descriptor,
    library_path,
    load_library,
    merge,
    moe_topk_softmax,
    pick_num_segments,
    pick_num_splits,
    pick_num_splits_multi,
    prefill,
    split_bounds,
    validate_kv_host,
)
