"""Paged attention over a block-table KV cache for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/pa.h`` (``libpa.so``, built in-tree by ``build.build()``); this
package only marshals torch tensors into those calls.
"""

from ._native import load  # noqa: F401
from .api import (  # noqa: F401
    BlockManager,
    PaError,
    kv_cache_struct,
    pa_copy_blocks,
    pa_decode,
    pa_decode_balanced,
    pa_decode_balanced_workspace_bytes,
    pa_decode_splitk,
    pa_lse_merge,
    pa_rope_write_kv,
    pa_splitk_num_splits,
    pa_splitk_workspace_bytes,
    pa_status_str,
    pa_varlen,
    pa_varlen_workspace_bytes,
    pa_write_decode_balanced,
    pa_write_decode_balanced_noalloc,
    pa_write_kv,
)
from .validate import PaMetadataError, validate_metadata  # noqa: F401
