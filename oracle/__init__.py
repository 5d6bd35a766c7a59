"""Float64 CPU oracle for paged decode attention and the KV-cache scatter.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library and its Python
binding (``paged_kv_cache_291_amd``) never import it, and this package imports
nothing from them: the two sides share no code.  The seeded input generators
(``paged_kv_cache_291_amd.workloads``) hold none of the method's arithmetic and
are the only thing both sides are fed from.

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself (a dense library routine, brute force in pure Python, closed forms,
invariants).  No function here is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    decode_values,
    kv_head_of,
    gather_rows,
    softmax_attention,
    paged_decode_ref,
    paged_decode_probs_ref,
    paged_decode_partials_ref,
    lse_combine_ref,
    reshape_and_cache_ref,
    copy_blocks_ref,
    e4m3_value,
    E4M3_VALUES,
    quantize_e4m3_ref,
    reshape_and_cache_fp8_ref,
    paged_prefill_ref,
)
from .block_manager import (  # noqa: F401
    BlockManagerRef,
    BlockManagerError,
    InvalidArg,
    NoBlocks,
    Capacity,
    blocks_for,
)
