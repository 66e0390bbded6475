"""MI355X-native indexer-driven top-k sparse attention with index reuse.

The library ``libsparse_attn.so`` (HIP, gfx950) exports a C ABI
(``include/sparse_attn.h``): ``sparse_index_score``, ``sparse_topk_select``
and ``sparse_attn_gather_fwd``.  This package is its thin Python binding plus
the host-side drivers that chain the calls for one step of each workload
(index reuse is simply passing the same index tensor to several attention
calls).
"""
from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    Cache,
    Rows,
    SAError,
    abi_version,
    attn_gather_fwd,
    attn_score,
    check_indices,
    index_score,
    load,
    topk_select,
)
