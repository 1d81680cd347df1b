"""cosa_proxy_ordered_mask_no_alloc against cosa_proxy_ordered_mask.

The no-allocation entry point keeps the proxy's pooled-key workspace in the
library's static device array; its masks (and exported scores) must equal,
bit for bit, those of the entry point that takes a caller's workspace.  Two
calls in a row: the first at the array's maximum size (four 128K sequences,
8 KV heads, head_dim 128: exactly 32 MiB of pooled keys), the second a
smaller ragged batch that runs over the first call's leftovers.
"""
import numpy as np
import pytest

import block_sparse_long_kap_amd as bk
import cosa_inputs as ci
from block_sparse_long_kap_amd import _lib

from .parity import report, upload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    ("stress", {}, 0.1),
    ("tiny", dict(seqlens=(1, 63, 64, 65, 200, 383), num_q_heads=8, num_kv_heads=2,
                  head_dim=128, q_block=128, shuffled_pages=True, spare_pages=7,
                  precision="bf16"), 0.3),
]


def test_no_alloc_proxy_equals_workspace_proxy_twice():
    for name, kw, budget in CASES:
        w = ci.get(name).with_(**kw) if kw else ci.get(name)
        print(f"[case] no-alloc proxy {name} {kw} budget={budget}", flush=True)
        x = ci.make(w).bf16_rounded()
        prob, q, k, _ = upload(x, DEV)
        need = prob.kap_workspace_size()
        assert 0 < need <= _lib.NO_ALLOC_SCRATCH_BYTES
        ref = bk.proxy_ordered_mask(prob, q, k, budget, debug=True)
        # outputs allocated up front: the call itself allocates nothing
        got = bk.proxy_ordered_mask(prob, q, k, budget, debug=True)
        for t in (got.blocks, got.pages, got.counts, got.hrm_counts):
            t.fill_(-7)
        got.debug_w.fill_(-1.0)
        got.debug_hrm.fill_(7)
        torch.cuda.synchronize()
        bk.proxy_ordered_mask_no_alloc(prob, q, k, budget, debug=True, out=got)
        torch.cuda.synchronize()
        for a, b, what in ((ref.blocks, got.blocks, "blocks"), (ref.pages, got.pages, "pages"),
                           (ref.counts, got.counts, "counts"),
                           (ref.hrm_counts, got.hrm_counts, "hrm_counts"),
                           (ref.debug_w.view(torch.int32), got.debug_w.view(torch.int32), "w"),
                           (ref.debug_hrm, got.debug_hrm, "hrm")):
            assert torch.equal(a, b), f"{name}: {what} differ"
        report(f"no-alloc proxy {name}", workspace_bytes=need,
               rows=int(np.prod(ref.counts.shape)), kept=int(ref.counts.sum()))
