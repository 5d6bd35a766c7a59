"""MI355X-native paged decode attention: hand-written HIP for gfx950 behind a C ABI.

Entry points (same names as the C ABI in ``include/pagedattn.h``):
``paged_attention_decode``, ``reshape_and_cache``, ``pa_decode_workspace_size``,
``pa_status_string``.  Inputs are torch tensors on a HIP device; torch provides
memory and streams only.
"""

from ._binding import (  # noqa: F401
    DTYPE_CODES,
    EXPORTED,
    LIB_PATH,
    PA_FLAG_SHARED_BLOCKS,
    PagedAttnError,
    decode_workspace_bytes,
    load_library,
    pa_decode_workspace_size,
    pa_status_string,
    paged_attention_decode,
    reshape_and_cache,
)
