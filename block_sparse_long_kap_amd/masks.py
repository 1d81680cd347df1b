"""Mask format conversions on the device (torch tensor plumbing).

Used to set up the logical-skip comparison of ``cosa_block_mask_prefill``
from an ordered mask; not part of the sparse path itself.
"""
from __future__ import annotations

import torch

from .api import OrderedMask, Problem


def block_bitmask(problem: Problem, mask: OrderedMask) -> torch.Tensor:
    """int32 [B][Hq][NQB][words] bitmask (uint32 bit patterns) of the blocks an
    ordered mask keeps: bit j % 32 of word j / 32 is set iff block j is listed."""
    n_max = -(-problem.max_seqlen // problem.kv_block)
    words = -(-n_max // 32)
    rows = tuple(mask.blocks.shape[:-1])
    blocks = mask.blocks.long()
    sel = torch.zeros(rows + (words * 32,), dtype=torch.int64, device=blocks.device)
    # the listed blocks of a row are distinct; padding (-1) adds 0 to block 0
    sel.scatter_add_(-1, blocks.clamp(min=0), (blocks >= 0).long())
    weights = torch.ones(32, dtype=torch.int64, device=blocks.device) << torch.arange(
        32, device=blocks.device)
    packed = (sel.view(rows + (words, 32)) * weights).sum(-1)       # [0, 2^32)
    packed = packed - ((packed >> 31) << 32)                         # as int32 bits
    return packed.to(torch.int32).contiguous()
