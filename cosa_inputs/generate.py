"""Seeded synthetic inputs for paged causal prefill attention.

Produces queries, a paged KV pool and per-sequence page tables for one
attention layer.  Both the GPU path and the CPU oracle consume the arrays made
here; the module holds no attention, pooling, scoring or selection arithmetic,
only random draws, planted structure and layout.

Layout (identical to the one the C ABI documents):

* ``q``          float32 ``[T][Hq][D]`` packed over sequences (T = sum of lengths)
* ``k_pool``     float32 ``[P][Hkv][page][D]``  (one page holds ``page`` tokens)
* ``v_pool``     float32 ``[P][Hkv][page][D]``
* ``page_table`` int32   ``[B][max_pages]`` logical block -> physical page, -1 unused
* ``cu_seqlens`` int32   ``[B+1]`` prefix sums of the sequence lengths

Spare pages of the pool and the unused tail slots of each sequence's last page
are filled with NaN, so that any read the causal mask should exclude shows up
as a non-finite output.

Random streams: ``numpy.random.Generator(PCG64)`` seeded from
``SeedSequence(seed)`` and spawned into six streams in the order
[Q, K, V, structure, pages, head-mix].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

from .configs import HeadPattern, Workload


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray            # float32 [T][Hq][D]
    k_pool: np.ndarray       # float32 [P][Hkv][page][D]
    v_pool: np.ndarray       # float32 [P][Hkv][page][D]
    page_table: np.ndarray   # int32 [B][max_pages]
    cu_seqlens: np.ndarray   # int32 [B+1]
    head_patterns: Tuple[HeadPattern, ...]   # per (b * Hkv + g)

    @property
    def seqlens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    def bf16_rounded(self) -> "Inputs":
        """Copy with q, k_pool and v_pool rounded to bfloat16 (round to
        nearest even), still stored as float32 so that every later widening
        to float64 is exact."""
        return Inputs(self.workload, round_to_bf16(self.q), round_to_bf16(self.k_pool),
                      round_to_bf16(self.v_pool), self.page_table.copy(),
                      self.cu_seqlens.copy(), self.head_patterns)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32; NaN stays NaN.  Uses torch's conversion when available, else
    the bit-level rule: add 0x7FFF plus the lowest kept bit, clear the low 16
    bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & 1)) & np.uint32(0xFFFF0000)
    r[nan] = 0x7FC00000
    return r.view(np.float32)


def _unit(rng: np.random.Generator, d: int, n: Optional[int] = None) -> np.ndarray:
    shape = (d,) if n is None else (n, d)
    v = rng.standard_normal(shape)
    v /= np.linalg.norm(v, axis=-1, keepdims=True)
    return v.astype(np.float32)


def _head_patterns(w: Workload, rng_mix: np.random.Generator) -> List[HeadPattern]:
    if w.pattern_mix is None:
        return [w.pattern] * w.num_kv_heads
    counts = [int(round(f * w.num_kv_heads)) for f, _ in w.pattern_mix]
    counts[0] += w.num_kv_heads - sum(counts)
    pats: List[HeadPattern] = []
    for c, (_, p) in zip(counts, w.pattern_mix):
        pats += [p] * c
    order = rng_mix.permutation(len(pats))
    return [pats[i] for i in order]


def _normals(stream: np.random.Generator, n_streams: int, shape) -> np.ndarray:
    """i.i.d. N(0,1) float32 array ``[n_streams, *shape]``, one spawned child
    stream per leading index, filled by a thread pool (the values do not
    depend on the number of threads)."""
    children = stream.bit_generator.seed_seq.spawn(n_streams)
    out = np.empty((n_streams,) + tuple(shape), dtype=np.float32)

    def fill(i):
        np.random.Generator(np.random.PCG64(children[i])).standard_normal(
            out[i].shape, dtype=np.float32, out=out[i])

    workers = max(1, min(n_streams, len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(n_streams)))
    return out


def _to_token_major(x: np.ndarray) -> np.ndarray:
    """[H][T][D] -> contiguous [T][H][D]."""
    try:
        import torch
        return torch.from_numpy(x).permute(1, 0, 2).contiguous().numpy()
    except ImportError:  # pragma: no cover
        return np.ascontiguousarray(x.transpose(1, 0, 2))


def make(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one layer's inputs for workload ``w`` (seed defaults to w.seed)."""
    seed = w.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rs, rp, rm = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]
    B, Hq, Hkv, D, PG = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    lens = np.asarray(w.seqlens, dtype=np.int64)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])

    q_h = _normals(rq, Hq, (T, D))        # head-major while structure is planted
    k_h = _normals(rk, Hkv, (T, D))
    v_h = _normals(rv, Hkv, (T, D))

    base_patterns = _head_patterns(w, rm)
    outlier_ch = None
    if w.outlier_channels > 0:
        outlier_ch = np.sort(rs.choice(D, size=w.outlier_channels, replace=False))

    patterns: List[HeadPattern] = []
    for b in range(B):
        L = int(lens[b])
        t0 = int(cu[b])
        nkb = (L + PG - 1) // PG
        for g in range(Hkv):
            pat = base_patterns[g]
            patterns.append(pat)
            u = _unit(rs, D)
            qs = q_h[g * grp:(g + 1) * grp, t0:t0 + L, :]   # view [grp][L][D]
            ks = k_h[g, t0:t0 + L, :]                        # view [L][D]
            if L == 0:
                continue
            if pat.q_dir:
                qs += (w.q_dir_gain * u)[None, None, :]
            if pat.sink:
                ks[:min(PG, L)] += pat.sink_value() * u
            if pat.stripes > 0 and nkb > 1:
                n = min(pat.stripes, nkb - 1)
                blocks = rs.choice(np.arange(1, nkb), size=n, replace=False)
                for j in blocks:
                    ks[j * PG:min((j + 1) * PG, L)] += pat.strength * u
            if pat.band > 0:
                vb = _unit(rs, D, nkb)                       # one vector per KV block
                blk = np.arange(L) // PG
                qs += (pat.strength * vb[blk])[None, :, :]
                padded = np.concatenate([vb, np.zeros((pat.band, D), np.float32)], 0)
                win = np.zeros((nkb, D), np.float32)
                for delta in range(pat.band):
                    win += padded[delta:delta + nkb]
                ks += pat.strength * win[blk]
    if outlier_ch is not None:
        k_h[:, :, outlier_ch] *= w.outlier_scale

    q = _to_token_major(q_h)
    del q_h

    # ---- paging -------------------------------------------------------------
    npages = [(int(L) + PG - 1) // PG for L in lens]
    used = int(sum(npages))
    P = used + w.spare_pages
    perm = rp.permutation(P) if w.shuffled_pages else np.arange(P)
    # page-table rows cover whole logical blocks (unused entries stay -1)
    per_block = w.block // PG
    max_pages = max(-(-n // per_block) * per_block for n in npages) if npages else 0
    page_table = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    k_pool = np.full((P, Hkv, PG, D), np.nan, dtype=np.float32)
    v_pool = np.full((P, Hkv, PG, D), np.nan, dtype=np.float32)
    off = 0
    for b in range(B):
        L = int(lens[b])
        t0 = int(cu[b])
        for j in range(npages[b]):
            p = int(perm[off + j])
            page_table[b, j] = p
            a, e = j * PG, min((j + 1) * PG, L)
            k_pool[p, :, :e - a, :] = k_h[:, t0 + a:t0 + e, :]
            v_pool[p, :, :e - a, :] = v_h[:, t0 + a:t0 + e, :]
        off += npages[b]
    return Inputs(w, q, k_pool, v_pool, page_table, cu, tuple(patterns))
