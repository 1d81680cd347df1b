"""Ordered-Skipping Kernel (OSK) of CoSA, float64 (oracle side).

What the pages fix (CoSA (paperpeel) §3.3, §4.3, App. C.2, App. D.1):

* the kernel visits only the blocks of the ordered mask M_KAP, in its order,
  by remapping pages of the paged KV cache (physical jumping);
* for every visited block it forms the exact logits S = scale * Q K^T, which
  in-kernel skipping cannot avoid (§3.3, limitation L1);
* it keeps the online-softmax statistics (running max m, running sum l,
  accumulator O); a block whose logits are negligible against the running
  max skips its value-side work (§3.3, Eq. (5), whose body is not printed);
* the decision is one vote per 128-row query tile: every row must agree,
  so one row can veto the skip (§3.3, limitation L2.2 "bucket effect";
  App. D.1);
* visiting order does not change the result of online softmax (§3.2 order
  invariance P2), so the reordering is correctness-preserving.

Reading taken for the missing Eq. (5) (in nats, on scaled logits): with bm_r
the largest logit of row r in the block and m_r the running max before the
block, the block is skipped when ``bm_r < m_r - tau`` holds for every valid
row of the tile; ``tau < 0`` switches the skip off (App. D.1: Delta = -1
disables in-kernel skipping).  A skipped block contributes to neither the
numerator nor the denominator (only value-side work is removed, §3.3).  The
comparison is IEEE: -inf < -inf is false, so a row with no key seen yet
vetoes the skip.  Rows that see no key at all give out = 0, lse = -inf.

Length-adaptive threshold (§5.1 "Hyperparameters", App. D.1: "Delta / N"):
Delta / N is read as the bound on exp(bm_r - m_r), so a sequence of N tokens
gets tau = ln(N / Delta) nats.  In that mode the skip is on for every Delta
> 0, whatever the sign of tau (a sequence shorter than Delta skips every
block that does not raise some row's max by more than ln(Delta / N)), and
off for Delta <= 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .dense import attention_rows
from .paging import materialise, sequence_slices


@dataclass
class TileResult:
    out: np.ndarray       # [n_rows][D]
    lse: np.ndarray       # [n_rows]
    skipped: np.ndarray   # [k] bool, per visited slot
    margin: np.ndarray    # [k] max over rows of (bm - m_prev + tau); skip iff < 0


def _block_logits(q_rows, row_pos, k, j, kv_block, scale):
    L = k.shape[0]
    a, e = j * kv_block, min((j + 1) * kv_block, L)
    s = scale * (q_rows @ k[a:e].T)                               # [n][e-a]
    s = np.where(np.arange(a, e)[None, :] <= row_pos[:, None], s, -np.inf)
    return s, a, e


def _row_margin(bm, m_prev, tau):
    """Per-row bm - m_prev + tau with the IEEE reading of -inf comparisons."""
    out = np.where(np.isneginf(m_prev), np.inf, bm - np.where(np.isneginf(m_prev), 0.0, m_prev) + tau)
    return np.where(np.isneginf(bm) & ~np.isneginf(m_prev), -np.inf, out)


def tau_from_delta(seqlen: int, delta: float) -> float:
    """tau = ln(N / Delta) nats for a sequence of N tokens (Delta > 0)."""
    return math.log(seqlen / delta)


def osk_tile_sequential(q_rows: np.ndarray, row_pos: np.ndarray, k: np.ndarray,
                        v: np.ndarray, blocks, tau: float, scale: float,
                        kv_block: int, skip_on: Optional[bool] = None) -> TileResult:
    """Visit ``blocks`` in order with the online softmax and the tile-wide skip.

    q_rows [n][D] are the valid query rows of one tile (positions row_pos),
    k, v [L][D] the sequence's keys and values for the matching KV head.
    ``skip_on`` defaults to ``tau >= 0``.
    """
    on = tau >= 0 if skip_on is None else skip_on
    n, D = q_rows.shape
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, D))
    skipped, margins = [], []
    for j in blocks:
        s, a, e = _block_logits(q_rows, row_pos, k, int(j), kv_block, scale)
        bm = s.max(axis=1)
        margin = float(np.max(_row_margin(bm, m, tau))) if n else -np.inf
        margins.append(margin)
        if on and np.all(bm < m - tau):
            skipped.append(True)
            continue
        skipped.append(False)
        m_new = np.maximum(m, bm)
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - np.where(np.isneginf(m), 0.0, m_new)))
        base = np.where(np.isneginf(m_new), 0.0, m_new)
        p = np.where(np.isneginf(m_new)[:, None], 0.0, np.exp(s - base[:, None]))
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[a:e]
        m = m_new
    has = l > 0
    out = np.where(has[:, None], o / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, np.where(np.isneginf(m), 0.0, m) + np.log(np.where(has, l, 1.0)), -np.inf)
    return TileResult(out, lse, np.asarray(skipped, dtype=bool), np.asarray(margins))


def osk_tile_closed_form(q_rows: np.ndarray, row_pos: np.ndarray, k: np.ndarray,
                         v: np.ndarray, blocks, tau: float, scale: float,
                         kv_block: int, skip_on: Optional[bool] = None) -> TileResult:
    """The same result without the sequential loop.

    A skipped block has bm_r < m_r - tau <= m_r for every row, so skipping never
    changes the running max: after slot t it is the prefix max of the block
    maxima whatever was skipped.  Hence slot t is skipped iff every row has
    bm_r(t) < max_{t' < t} bm_r(t') - tau, and the output is exact softmax
    attention restricted to the keys of the blocks that were not skipped
    (order invariance).
    """
    on = tau >= 0 if skip_on is None else skip_on
    n = q_rows.shape[0]
    L = k.shape[0]
    blocks = [int(j) for j in blocks]
    bms = np.stack([_block_logits(q_rows, row_pos, k, j, kv_block, scale)[0].max(axis=1)
                    for j in blocks]) if blocks else np.zeros((0, n))
    prev = np.full(n, -np.inf)
    skipped, margins = [], []
    for t in range(len(blocks)):
        margins.append(float(np.max(_row_margin(bms[t], prev, tau))) if n else -np.inf)
        skipped.append(on and bool(np.all(bms[t] < prev - tau)))
        prev = np.maximum(prev, bms[t])
    key_ok = np.zeros(L, dtype=bool)
    for j, sk in zip(blocks, skipped):
        if not sk:
            key_ok[j * kv_block:min((j + 1) * kv_block, L)] = True
    out, lse = attention_rows(q_rows, row_pos, k, v, scale, key_ok=key_ok)
    return TileResult(out, lse, np.asarray(skipped, dtype=bool), np.asarray(margins))


@dataclass
class PrefillResult:
    out: np.ndarray          # [T][Hq][D]
    lse: np.ndarray          # [Hq][T]
    skip_record: np.ndarray  # uint8 [B][Hq][NQBmax][C]
    margins: np.ndarray      # float64 [B][Hq][NQBmax][C] (nan past count)
    row_stats: np.ndarray    # int32 [B][Hq][NQBmax][2] (visited, skipped)


def osk_prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                page_table: np.ndarray, cu_seqlens: np.ndarray, num_kv_heads: int,
                q_block: int, kv_block: int, ordered_blocks: np.ndarray,
                counts: np.ndarray, tau: float, scale: float,
                closed_form: bool = False, tiles=None,
                delta: Optional[float] = None) -> PrefillResult:
    """OSK over a packed batch given an ordered mask in the C-ABI layout.

    ``tiles`` optionally restricts the work to a list of (b, h, i); outputs of
    other tiles stay zero.  With ``delta`` given, ``tau`` is ignored and each
    sequence b of length L_b uses tau_b = ln(L_b / delta), the skip being on
    iff delta > 0.
    """
    T, Hq, D = q.shape
    grp = Hq // num_kv_heads
    B, _, nqb_max, C = ordered_blocks.shape
    page_size = k_pool.shape[2]
    out = np.zeros((T, Hq, D))
    lse = np.full((Hq, T), -np.inf)
    rec = np.zeros((B, Hq, nqb_max, C), dtype=np.uint8)
    mar = np.full((B, Hq, nqb_max, C), np.nan)
    stats = np.zeros((B, Hq, nqb_max, 2), dtype=np.int32)
    want = None if tiles is None else set(tiles)
    fn = osk_tile_closed_form if closed_form else osk_tile_sequential
    for b, start, L in sequence_slices(cu_seqlens):
        if L == 0:
            continue
        if want is not None and not any(t[0] == b for t in want):
            continue
        if delta is None:
            tau_b, on = tau, tau >= 0
        else:
            on = delta > 0
            tau_b = tau_from_delta(L, delta) if on else -1.0
        keys = materialise(k_pool, page_table[b], L, page_size)
        vals = materialise(v_pool, page_table[b], L, page_size)
        nqb = (L + q_block - 1) // q_block
        for h in range(Hq):
            g = h // grp
            for i in range(nqb):
                if want is not None and (b, h, i) not in want:
                    continue
                rows = np.arange(i * q_block, min((i + 1) * q_block, L))
                cnt = int(counts[b, h, i])
                res = fn(np.asarray(q[start + rows, h, :], dtype=np.float64), rows,
                         keys[:, g, :], vals[:, g, :], ordered_blocks[b, h, i, :cnt],
                         tau_b, scale, kv_block, skip_on=on)
                out[start + rows, h, :] = res.out
                lse[h, start + rows] = res.lse
                rec[b, h, i, :cnt] = res.skipped
                mar[b, h, i, :cnt] = res.margin
                stats[b, h, i] = (cnt, int(res.skipped.sum()))
    return PrefillResult(out, lse, rec, mar, stats)


def dense_order_mask(cu_seqlens: np.ndarray, num_q_heads: int, q_block: int, kv_block: int):
    """Every causal candidate block of every tile in ascending order
    (stage-1 budget 100% without reordering), as (ordered_blocks, counts)."""
    B = len(cu_seqlens) - 1
    lens = np.diff(cu_seqlens)
    max_len = int(lens.max()) if B else 0
    nqb_max = max((max_len + q_block - 1) // q_block, 1)
    C = max((max_len + kv_block - 1) // kv_block, 1)
    blocks = np.full((B, num_q_heads, nqb_max, C), -1, dtype=np.int32)
    counts = np.zeros((B, num_q_heads, nqb_max), dtype=np.int32)
    for b in range(B):
        L = int(lens[b])
        for i in range((L + q_block - 1) // q_block):
            last = min((i + 1) * q_block, L) - 1
            n = last // kv_block + 1
            blocks[b, :, i, :n] = np.arange(n)
            counts[b, :, i] = n
    return blocks, counts
