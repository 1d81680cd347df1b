"""Kernel-Aware Proxy (KAP) of CoSA, float64 (oracle side).

What the pages fix (CoSA (paperpeel) §4.1, §4.2, App. C.1; researchpod
summary): for one query block the proxy gives every candidate key block an
importance score and a "have rowmax" (HRM) flag; it sorts the HRM group and
the non-HRM group independently by score, puts the HRM group first and keeps
the leading entries under the stage-1 budget.  The kept sequence, in that
order, is the computation-order mask M_KAP; blocks outside it are skipped by
the kernel without being visited (§4.1, block type 1).  Scoring and pooling
are one fused operation (§5.1 "Implementation details").

What the pages leave open (the body of §4.2 "Block ranking" is missing) and
the reading taken here:

* pooling: a query block (tile) of ``q_block`` rows is pooled into proxy rows
  of ``rows_per_proxy`` consecutive queries (16 by default); a key block of
  ``kv_block`` keys is pooled into one vector.  Pooling is the mean over the
  valid (in-sequence) rows or keys.
* score: ``s[r, j] = scale * <qbar_r, kbar_j>``.  By bilinearity this equals
  the mean of the exact logits over the (proxy row x key block) sub-block.
* candidates of proxy row r: key blocks whose first key is at or before the
  last query of the row (causal at block granularity, no forced blocks).
  Candidates of the tile: the union, ``n = last_row // kv_block + 1``.
* importance ``w_j``: softmax of ``s[r, :]`` over proxy row r's candidates,
  averaged over the tile's non-empty proxy rows (rows for which j is not a
  candidate contribute 0).
* HRM: j is flagged if it is the arg-max of ``s[r, :]`` for at least one
  proxy row r (ties to the lowest j).
* order: ascending by the key (not HRM, -w, j): HRM first, larger w first,
  then lower block index.
* budget: ``k = clamp(ceil(n * beta_ppm / 1e6), 1, n)`` in integers, with
  ``beta_ppm = floor(beta * 1e6 + 0.5)``; truncation happens after the two
  groups are concatenated, so an HRM block can displace a higher-w non-HRM
  block.
* KV-group-shared masks (one mask for the query heads that share a KV head,
  the GQA packing the pages leave to the implementation): the proxy rows of
  all the group's heads for the tile are scored together, w_j is their mean
  and HRM marks the arg-max block of any of them; the rest is unchanged.
* Top-p (§5.1 "Hyperparameters", App. D.1: stage-1 Top-p with p = 0.95):
  the importance scores of a tile sum to 1 (each proxy row's softmax sums to
  1 over its candidates), so they are read as the probability mass of the
  blocks; Top-p keeps the shortest prefix of the HRM-first order whose mass
  reaches p (at least one block; p = 1 keeps every candidate).  Combined
  with a budget the smaller of the two counts is kept.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .paging import materialise, sequence_slices

ROWS_PER_PROXY = 16


def budget_ppm(beta: float) -> int:
    """Stage-1 budget as an integer in parts per million."""
    if not (0.0 < beta <= 1.0):
        raise ValueError("budget must lie in (0, 1]")
    return int(np.floor(beta * 1e6 + 0.5))


def budget_count(n: int, beta_ppm: int) -> int:
    """Number of blocks kept out of n candidates: clamp(ceil(n*beta), 1, n)."""
    if n <= 0:
        return 0
    k = (n * beta_ppm + 999_999) // 1_000_000
    return max(1, min(n, k))


def top_p_count(w_in_order: np.ndarray, p: float) -> int:
    """Smallest k >= 1 whose first k importance scores (in visiting order) add
    up to at least p; every candidate when p >= 1 or when the sum never gets
    there."""
    if not (0.0 < p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")
    n = len(w_in_order)
    if n == 0:
        return 0
    if p >= 1.0:
        return n
    reached = np.flatnonzero(np.cumsum(w_in_order) >= p)
    return int(reached[0]) + 1 if reached.size else n


def mask_capacity(max_seqlen: int, kv_block: int, beta_ppm: int) -> int:
    """Entries per mask row: the largest k over all tiles of the batch."""
    n_max = (max_seqlen + kv_block - 1) // kv_block
    return budget_count(n_max, beta_ppm) if n_max > 0 else 1


def pooled_keys(k_g: np.ndarray, kv_block: int) -> np.ndarray:
    """kbar[j] = mean of the valid keys of key block j.  k_g: [L][D]."""
    L, D = k_g.shape
    nkb = (L + kv_block - 1) // kv_block
    out = np.zeros((nkb, D), dtype=np.float64)
    for j in range(nkb):
        out[j] = k_g[j * kv_block:min((j + 1) * kv_block, L)].mean(axis=0)
    return out


def pooled_queries(q_h: np.ndarray, q_block: int, rows_per_proxy: int = ROWS_PER_PROXY):
    """Proxy rows of every tile.

    Returns (qbar [NQB][R][D], last [NQB][R], valid [NQB][R]) where proxy row
    r of tile i covers positions [i*q_block + r*g, +g) within the sequence,
    qbar is the mean of its valid queries, ``last`` its last valid position
    and ``valid`` whether it holds any query.
    """
    L, D = q_h.shape
    R = q_block // rows_per_proxy
    nqb = (L + q_block - 1) // q_block
    qbar = np.zeros((nqb, R, D), dtype=np.float64)
    last = np.full((nqb, R), -1, dtype=np.int64)
    valid = np.zeros((nqb, R), dtype=bool)
    for i in range(nqb):
        for r in range(R):
            a = i * q_block + r * rows_per_proxy
            e = min(a + rows_per_proxy, L)
            if e > a:
                qbar[i, r] = q_h[a:e].mean(axis=0)
                last[i, r] = e - 1
                valid[i, r] = True
    return qbar, last, valid


@dataclass
class TileProxy:
    scores: np.ndarray      # [R_i][n] scaled pooled logits (-inf off-candidate)
    probs: np.ndarray       # [R_i][n] per-proxy-row softmax over its candidates
    w: np.ndarray           # [n] importance
    hrm: np.ndarray         # [n] bool
    order: np.ndarray       # [n] full flag-grouped order (block ids)
    k: int                  # kept count
    n: int                  # candidate count

    @property
    def blocks(self) -> np.ndarray:
        return self.order[:self.k]

    @property
    def hrm_count(self) -> int:
        return int(self.hrm[self.blocks].sum())


def score_tile(qbar: np.ndarray, last: np.ndarray, kbar: np.ndarray, scale: float,
               kv_block: int):
    """Scores, per-row softmax, importance and HRM flags of one tile.

    qbar [R_i][D] and last [R_i] describe the tile's non-empty proxy rows.
    """
    n = int(last.max()) // kv_block + 1
    s = scale * (qbar @ kbar[:n].T)                                 # [R_i][n]
    cand = np.arange(n)[None, :] <= (last // kv_block)[:, None]
    s = np.where(cand, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    w = p.sum(axis=0) / qbar.shape[0]
    hrm = np.zeros(n, dtype=bool)
    hrm[np.argmax(s, axis=1)] = True                                # lowest j on ties
    return s, p, w, hrm


def flag_grouped_order(w: np.ndarray, hrm: np.ndarray) -> np.ndarray:
    """All candidates sorted by (not HRM, -w, j) ascending."""
    j = np.arange(len(w))
    return np.lexsort((j, -w, (~hrm).astype(np.int64)))


def kap_tile(qbar: np.ndarray, last: np.ndarray, kbar: np.ndarray, scale: float,
             kv_block: int, beta_ppm: int, top_p=None) -> TileProxy:
    s, p, w, hrm = score_tile(qbar, last, kbar, scale, kv_block)
    order = flag_grouped_order(w, hrm)
    n = len(w)
    k = budget_count(n, beta_ppm)
    if top_p is not None:
        k = min(k, top_p_count(w[order], top_p))
    return TileProxy(s, p, w, hrm, order, k, n)


def head_tiles(q_h: np.ndarray, k_g: np.ndarray, scale: float, q_block: int,
               kv_block: int, beta_ppm: int, rows_per_proxy: int = ROWS_PER_PROXY,
               tiles=None, top_p=None):
    """KAP for every tile (or the listed tiles) of one (sequence, query head)."""
    kbar = pooled_keys(k_g, kv_block)
    qbar, last, valid = pooled_queries(q_h, q_block, rows_per_proxy)
    idx = range(qbar.shape[0]) if tiles is None else tiles
    return {i: kap_tile(qbar[i][valid[i]], last[i][valid[i]], kbar, scale, kv_block,
                        beta_ppm, top_p) for i in idx}


def group_tiles(q_heads, k_g: np.ndarray, scale: float, q_block: int, kv_block: int,
                beta_ppm: int, rows_per_proxy: int = ROWS_PER_PROXY, tiles=None, top_p=None):
    """KAP for every tile (or the listed tiles) of one (sequence, KV head) with
    one mask shared by the group's query heads ``q_heads`` (a list of [L][D]
    arrays): the proxy rows of every head for the tile are scored together."""
    kbar = pooled_keys(k_g, kv_block)
    pooled = [pooled_queries(qh, q_block, rows_per_proxy) for qh in q_heads]
    nqb = pooled[0][0].shape[0]
    idx = range(nqb) if tiles is None else tiles
    out = {}
    for i in idx:
        qbar = np.concatenate([qb[i][va[i]] for qb, _, va in pooled], axis=0)
        last = np.concatenate([la[i][va[i]] for _, la, va in pooled], axis=0)
        out[i] = kap_tile(qbar, last, kbar, scale, kv_block, beta_ppm, top_p)
    return out


@dataclass
class OrderedMask:
    blocks: np.ndarray      # int32 [B][Hq][NQBmax][C], -1 past count
    pages: np.ndarray       # int32 [B][Hq][NQBmax][C * kv_block / page], -1 past count
    counts: np.ndarray      # int32 [B][Hq][NQBmax]
    hrm_counts: np.ndarray  # int32 [B][Hq][NQBmax]
    capacity: int
    tiles: dict             # (b, h, i) -> TileProxy


def proxy_ordered_mask(q: np.ndarray, k_pool: np.ndarray, page_table: np.ndarray,
                       cu_seqlens: np.ndarray, num_kv_heads: int, q_block: int,
                       kv_block: int, budget: float, scale: float,
                       rows_per_proxy: int = ROWS_PER_PROXY, top_p=None,
                       shared_kv: bool = False) -> OrderedMask:
    """M_KAP for a packed batch, in the layout of the C ABI.

    q [T][Hq][D], k_pool [P][Hkv][page][D] (bf16-exact values, any float
    dtype), page_table [B][max_pages], cu_seqlens [B+1].  With ``top_p`` the
    kept count is the smaller of the budget count and the Top-p count; the
    capacity stays the budget's.  With ``shared_kv`` there is one mask row
    per (sequence, KV head, tile): arrays are [B][Hkv][NQBmax](...).
    """
    T, Hq, D = q.shape
    grp = Hq // num_kv_heads
    beta_ppm = budget_ppm(budget)
    B = len(cu_seqlens) - 1
    max_len = int(np.max(np.diff(cu_seqlens))) if B > 0 else 0
    nqb_max = max((max_len + q_block - 1) // q_block, 1)
    C = mask_capacity(max_len, kv_block, beta_ppm)
    H = num_kv_heads if shared_kv else Hq
    blocks = np.full((B, H, nqb_max, C), -1, dtype=np.int32)
    page_size = k_pool.shape[2]
    if kv_block % page_size != 0:
        raise ValueError("a logical key block must span whole pages")
    ppb = kv_block // page_size
    pages = np.full((B, H, nqb_max, C * ppb), -1, dtype=np.int32)
    counts = np.zeros((B, H, nqb_max), dtype=np.int32)
    hrm_counts = np.zeros((B, H, nqb_max), dtype=np.int32)
    tiles = {}
    for b, start, L in sequence_slices(cu_seqlens):
        if L == 0:
            continue
        keys = materialise(k_pool, page_table[b], L, page_size)        # [L][Hkv][D]
        for h in range(H):
            if shared_kv:
                res = group_tiles([np.asarray(q[start:start + L, hh, :], dtype=np.float64)
                                   for hh in range(h * grp, (h + 1) * grp)],
                                  keys[:, h, :], scale, q_block, kv_block, beta_ppm,
                                  rows_per_proxy, top_p=top_p)
            else:
                res = head_tiles(np.asarray(q[start:start + L, h, :], dtype=np.float64),
                                 keys[:, h // grp, :], scale, q_block, kv_block, beta_ppm,
                                 rows_per_proxy, top_p=top_p)
            for i, tp in res.items():
                kk = tp.k
                blocks[b, h, i, :kk] = tp.blocks
                for t, j in enumerate(tp.blocks):
                    for e in range(ppb):   # pages of the block that hold keys
                        if j * kv_block + e * page_size < L:
                            pages[b, h, i, t * ppb + e] = page_table[b][j * ppb + e]
                counts[b, h, i] = kk
                hrm_counts[b, h, i] = tp.hrm_count
                tiles[(b, h, i)] = tp
    return OrderedMask(blocks, pages, counts, hrm_counts, C, tiles)
