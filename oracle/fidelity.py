"""Proxy fidelity: the KAP kept set against the exact attention mass, float64.

CoSA (paperpeel) §3.2 (the P1 "proxy fidelity" observation, Fig. 2) measures
how well a proxy's block mask matches the mask an oracle would pick from the
exact attention, by IoU at a matched budget, and finds that fidelity drops as
the budget tightens.  The pages give neither the exact attention-side
selection nor the averaging; the plainest reading is taken:

* exact mass of key block j for query tile i: the mean over the tile's valid
  rows t of sum_{u in block j, u <= t} softmax_u(scale * <Q_t, K_u>), i.e.
  the share of the tile's attention probability that falls in block j (the
  masses of a tile sum to 1);
* exact mask at a matched budget: the k blocks of largest exact mass, k being
  the count the proxy kept for that tile (ties to the lower block index);
* IoU = |A n B| / |A u B|; mass recall = the exact mass covered by a set.

Used only by tests (a CPU report of IoU against budget on synthetic inputs).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .kap import budget_ppm, head_tiles


def exact_block_mass(q_rows: np.ndarray, row_pos: np.ndarray, k: np.ndarray, scale: float,
                     kv_block: int) -> np.ndarray:
    """Mean causal softmax probability per key block over the given rows.

    q_rows [n][D], row_pos [n], k [L][D].  Returns [ceil((max pos + 1) / kv_block)].
    """
    L = k.shape[0]
    n_blocks = int(row_pos.max()) // kv_block + 1
    s = scale * (q_rows @ k.T)                                    # [n][L]
    s = np.where(np.arange(L)[None, :] <= row_pos[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    mass = np.zeros(n_blocks)
    for j in range(n_blocks):
        mass[j] = p[:, j * kv_block:min((j + 1) * kv_block, L)].sum(axis=1).mean()
    return mass


def top_mass_blocks(mass: np.ndarray, k: int) -> np.ndarray:
    """The k blocks of largest mass, ties to the lower block index."""
    order = np.lexsort((np.arange(len(mass)), -mass))
    return order[:k]


def iou(a, b) -> float:
    a, b = set(int(x) for x in a), set(int(x) for x in b)
    union = a | b
    return len(a & b) / len(union) if union else 1.0


@dataclass
class FidelityRow:
    budget: float
    tiles: int
    mean_iou: float
    proxy_mass: float    # mean exact mass covered by the proxy's kept set
    oracle_mass: float   # mean exact mass covered by the exact top-k set


def proxy_fidelity(q_h: np.ndarray, k_g: np.ndarray, scale: float, q_block: int,
                   kv_block: int, budgets, tiles=None) -> list:
    """IoU and mass recall of the KAP kept set against the exact top-k blocks
    for one (sequence, query head), per budget, over ``tiles`` (default all)."""
    L = q_h.shape[0]
    nqb = (L + q_block - 1) // q_block
    idx = list(range(nqb)) if tiles is None else list(tiles)
    masses = {}
    for i in idx:
        rows = np.arange(i * q_block, min((i + 1) * q_block, L))
        masses[i] = exact_block_mass(q_h[rows], rows, k_g, scale, kv_block)
    out = []
    for beta in budgets:
        res = head_tiles(q_h, k_g, scale, q_block, kv_block, budget_ppm(beta), tiles=idx)
        ious, pm, om = [], [], []
        for i, t in res.items():
            exact = top_mass_blocks(masses[i], t.k)
            ious.append(iou(t.blocks, exact))
            pm.append(masses[i][t.blocks].sum())
            om.append(masses[i][exact].sum())
        out.append(FidelityRow(beta, len(ious), float(np.mean(ious)), float(np.mean(pm)),
                               float(np.mean(om))))
    return out
