"""CoSA block-sparse prefill attention for MI355X (gfx950).

The compute lives in ``libcosa.so`` (hand-written HIP kernels behind the C ABI
of ``include/cosa.h``); this package is its thin Python binding.  Importing it
does not load the library; the first call does, and raises if the library has
not been built (``python -m block_sparse_long_kap_amd.build``).
"""
from .api import (KapWorkspace, OrderedMask, PrefillOutput, Problem,  # noqa: F401
                  block_mask_prefill, dense_prefill, osk_prefill, osk_prefill_delta,
                  osk_prefill_shared_kv,
                  proxy_ordered_mask, proxy_ordered_mask_no_alloc,
                  proxy_ordered_mask_shared_kv, proxy_ordered_mask_top_p,
                  sparse_prefill)
