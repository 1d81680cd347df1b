"""Host check of the ordered-mask -> block-bitmask conversion (torch on the CPU)."""
import numpy as np
import torch

import block_sparse_long_kap_amd as bk
from block_sparse_long_kap_amd.masks import block_bitmask


def test_bitmask_matches_listed_blocks():
    rng = np.random.default_rng(0)
    L, n_max = 3000, 47                      # 47 blocks -> 2 words per row
    cu = torch.tensor([0, L], dtype=torch.int32)
    pt = torch.arange(n_max, dtype=torch.int32).reshape(1, n_max)
    prob = bk.Problem(cu_seqlens=cu, page_table=pt, num_q_heads=2, num_kv_heads=1, head_dim=64,
                      max_seqlen=L, total_q=L, num_pages=n_max)
    nqb = -(-L // 128)
    C = 40
    blocks = np.full((1, 2, nqb, C), -1, dtype=np.int32)
    for h in range(2):
        for i in range(nqb):
            n = min((i + 1) * 128, L) // 64 + 1 if (i + 1) * 128 <= L else (L - 1) // 64 + 1
            k = int(rng.integers(1, min(n, C) + 1))
            blocks[0, h, i, :k] = rng.choice(n, size=k, replace=False)
    mask = bk.OrderedMask(blocks=torch.from_numpy(blocks), pages=torch.from_numpy(blocks),
                          counts=torch.from_numpy((blocks >= 0).sum(-1).astype(np.int32)),
                          hrm_counts=None, capacity=C)
    bits = block_bitmask(prob, mask).numpy().view(np.uint32)
    assert bits.shape == (1, 2, nqb, 2)
    for idx in np.ndindex(1, 2, nqb):
        want = set(int(j) for j in blocks[idx] if j >= 0)
        got = {j for j in range(64) if (int(bits[idx][j // 32]) >> (j % 32)) & 1}
        assert got == want, idx
