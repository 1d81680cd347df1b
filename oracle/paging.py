"""De-paging of a paged KV cache (oracle side).

The KV cache is stored in fixed-size pages that need not be contiguous, with a
per-sequence page table mapping logical block j to a physical page (CoSA
(paperpeel), §3.2 last paragraph and §4.3 "Any-order page visiting"; the
layout follows PagedAttention, which the paper builds on).

Pool layout: ``pool[page][kv_head][slot][dim]``; token t of a sequence lives
in page ``page_table[t // page_size]`` at slot ``t % page_size``.
"""
from __future__ import annotations

import numpy as np


def materialise(pool: np.ndarray, page_table_row: np.ndarray, length: int,
                page_size: int) -> np.ndarray:
    """Return the sequence's keys (or values) as float64 ``[L][H][D]``.

    Only the first ``length`` tokens are read; pool slots past the end of
    the sequence (and pages the table does not name) are never touched.
    """
    n_pages = (length + page_size - 1) // page_size
    if length == 0:
        return np.zeros((0, pool.shape[1], pool.shape[3]), dtype=np.float64)
    pages = pool[np.asarray(page_table_row[:n_pages], dtype=np.int64)]  # [n][H][page][D]
    tokens = pages.transpose(0, 2, 1, 3).reshape(n_pages * page_size, pool.shape[1],
                                                 pool.shape[3])
    return np.array(tokens[:length], dtype=np.float64)


def sequence_slices(cu_seqlens: np.ndarray):
    """Yield (b, start, length) for every sequence of a packed batch."""
    for b in range(len(cu_seqlens) - 1):
        s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        yield b, s, e - s
