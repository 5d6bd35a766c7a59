"""MI355X-native paged decode attention: hand-written HIP for gfx950 behind a C ABI.

Entry points (same names as the C ABI in ``include/pagedattn.h``):
``paged_attention_decode``, ``reshape_and_cache``, ``paged_attention_decode_fp8``,
``reshape_and_cache_fp8``, ``paged_attention_prefill``, ``copy_blocks``,
``pa_decode_workspace_size``, ``pa_status_string``, and ``BlockManager``
over the host block manager (``pa_bm_*``).  Inputs of the device calls are
torch tensors on a HIP device; torch provides memory and streams only.
"""

from ._binding import (  # noqa: F401
    DTYPE_CODES,
    EXPORTED,
    LIB_PATH,
    PA_ERR_CAPACITY,
    PA_ERR_INVALID_ARG,
    PA_ERR_NO_BLOCKS,
    PA_ERR_SCRATCH,
    PA_FLAG_SHARED_BLOCKS,
    PA_FP8_E4M3,
    BlockManager,
    PagedAttnError,
    copy_blocks,
    decode_workspace_bytes,
    load_library,
    pa_decode_workspace_size,
    pa_prefill_workspace_size,
    pa_status_string,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_decode_fp8,
    paged_attention_prefill,
    reshape_and_cache,
    reshape_and_cache_fp8,
)
