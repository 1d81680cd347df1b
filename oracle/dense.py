"""Dense causal softmax attention, float64 (oracle side).

CoSA (paperpeel) §3.1 "Dense Attention" has its heading only; the full
attention baseline of §5.1 is FlashAttention-2, which computes the textbook
causal attention written out here:

    out_q = sum_{u <= q} softmax_u(scale * <Q_q, K_u>) V_u
    lse_q = log sum_{u <= q} exp(scale * <Q_q, K_u>)

Grouped-query attention: query head h reads KV head h // (Hq / Hkv).
Rows are processed in chunks only to bound memory; each row's softmax is
computed whole, exactly as the definition states.
"""
from __future__ import annotations

import numpy as np


def attention_rows(q_rows: np.ndarray, row_pos: np.ndarray, k: np.ndarray,
                   v: np.ndarray, scale: float, key_ok: np.ndarray | None = None):
    """Causal softmax attention for a set of query rows of one head.

    q_rows  [n][D]   queries (float64)
    row_pos [n]      their positions in the sequence
    k, v    [L][D]   keys / values of the sequence for the matching KV head
    key_ok  [L] bool optional extra key filter (keys with False are excluded)

    Returns (out [n][D], lse [n]).  A row that sees no key gets out = 0 and
    lse = -inf.
    """
    L = k.shape[0]
    s = scale * (q_rows @ k.T)                                   # [n][L]
    allowed = np.arange(L)[None, :] <= row_pos[:, None]
    if key_ok is not None:
        allowed = allowed & key_ok[None, :]
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1) if L > 0 else np.full(len(q_rows), -np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.exp(s - m_safe[:, None])                               # exp(-inf) = 0
    l = e.sum(axis=1)
    out = np.where(has[:, None], (e @ v) / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                           row_chunk: int = 512):
    """Causal attention for one sequence.

    q [L][Hq][D], k/v [L][Hkv][D] (float64).  Returns out [L][Hq][D] and
    lse [Hq][L].
    """
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    out = np.zeros((L, Hq, D), dtype=np.float64)
    lse = np.full((Hq, L), -np.inf, dtype=np.float64)
    for h in range(Hq):
        g = h // grp
        kg, vg = k[:, g, :], v[:, g, :]
        for a in range(0, L, row_chunk):
            e = min(a + row_chunk, L)
            pos = np.arange(a, e)
            # only keys <= the last row of the chunk can contribute
            o, ls = attention_rows(q[a:e, h, :], pos, kg[:e], vg[:e], scale)
            out[a:e, h, :] = o
            lse[h, a:e] = ls
    return out, lse
