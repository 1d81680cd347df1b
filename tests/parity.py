"""Helpers for GPU-vs-oracle parity tests.

Expected values always come from the CPU oracle (``oracle/``) run on the same
seeded, bf16-rounded inputs; GPU results are only ever the thing checked.
Where the method allows several correct answers (near-ties of the float
ranking, skip decisions within rounding of the threshold), the checks
enumerate the alternatives on the oracle side and require the GPU result to
be one of them, counting such cases.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field

import numpy as np

from oracle import dense as odense
from oracle.kap import TileProxy

# spec tolerances for bf16 inputs on the same visited set
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# skip decisions closer than this (nats) to the threshold may go either way
MARGIN_TOL = 1e-3
# KAP near-ties: relative gap of importance scores, absolute gap of proxy logits
W_RTOL = 1e-4
HRM_GAP = 1e-4

# One line per parity check with its tallies (exact rows, near-ties,
# near-threshold slots ...), printed again in the terminal summary by
# tests/conftest.py so that a quiet run still shows them.
SUMMARY: list = []


def report(label: str, **counts) -> None:
    line = f"{label}: " + " ".join(f"{k}={v}" for k, v in counts.items())
    SUMMARY.append(line)
    print(f"[parity] {line}", flush=True)


def selection_on_own_scores(w32, hrm, n, beta_ppm, top_p=1.0):
    """The documented selection rule applied to a kernel's own exported fp32
    importance scores and HRM flags: HRM-first order (w descending, block
    ascending inside each group), budget count, and with top_p < 1 the Top-p
    count over w rounded down to 2^-48 (p likewise).  The kernel's mask must
    equal this bit for bit."""
    from oracle import kap as okap
    w32 = np.asarray(w32[:n], dtype=np.float32)
    order = okap.flag_grouped_order(w32.astype(np.float64), np.asarray(hrm[:n], dtype=bool))
    k = okap.budget_count(n, beta_ppm)
    if top_p < 1.0:
        fx = np.floor(w32.astype(np.float64) * 2.0 ** 48).astype(np.int64)
        target = int(np.floor(np.float64(np.float32(top_p)) * 2.0 ** 48))
        cum = np.cumsum(fx[order])
        hit = np.flatnonzero(cum >= target)
        k = min(k, int(hit[0]) + 1 if hit.size else n)
    return order[:k]


def upload(x, device, q_block=None):
    """Seeded inputs (bf16-rounded float32 numpy) -> device tensors + Problem."""
    import torch

    from block_sparse_long_kap_amd import Problem
    w = x.workload
    q = torch.from_numpy(x.q).to(torch.bfloat16).to(device)
    k = torch.from_numpy(x.k_pool).to(torch.bfloat16).to(device)
    v = torch.from_numpy(x.v_pool).to(torch.bfloat16).to(device)
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(device)
    pt = torch.from_numpy(x.page_table.astype(np.int32)).to(device)
    prob = Problem(cu_seqlens=cu, page_table=pt, num_q_heads=w.num_q_heads,
                   num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                   max_seqlen=int(max(w.seqlens)), total_q=int(x.cu_seqlens[-1]),
                   num_pages=x.k_pool.shape[0], q_block=q_block or w.q_block,
                   page_size=w.page_size, softmax_scale=w.softmax_scale, kv_block=w.block)
    return prob, q, k, v


@dataclass
class ErrStats:
    max_abs: float = 0.0
    sum_abs: float = 0.0
    count: int = 0
    notes: list = field(default_factory=list)

    def add(self, gpu: np.ndarray, ref: np.ndarray):
        assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
        assert np.all(np.isfinite(gpu)), "non-finite GPU output"
        d = np.abs(gpu.astype(np.float64) - ref)
        if d.size:
            self.max_abs = max(self.max_abs, float(d.max()))
            self.sum_abs += float(d.sum())
            self.count += d.size

    @property
    def mean_abs(self) -> float:
        return self.sum_abs / max(self.count, 1)

    def assert_ok(self, max_abs=MAX_ABS, mean_abs=MEAN_ABS, label=""):
        print(f"[parity] {label}: max_abs={self.max_abs:.3e} mean_abs={self.mean_abs:.3e} "
              f"elements={self.count}")
        assert self.max_abs <= max_abs, f"{label}: max abs error {self.max_abs} > {max_abs}"
        assert self.mean_abs <= mean_abs, f"{label}: mean abs error {self.mean_abs} > {mean_abs}"


# ---------------------------------------------------------------------------
# KAP mask rows


def _hrm_sets(tile: TileProxy, gap: float):
    certain, possible = set(), set()
    for row in tile.scores:
        fin = np.isfinite(row)
        mx = row[fin].max()
        near = np.flatnonzero(fin & (row >= mx - gap))
        if len(near) == 1:
            certain.add(int(near[0]))
        possible.update(int(j) for j in near)
    return certain, possible


def expected_pages(blocks, page_table_row, ppb=1, kv_block=None, L=None):
    """The page list of an ordered block list: P = ppb pages per block, -1 for
    a page past the sequence's end."""
    out = []
    for j in np.asarray(blocks, dtype=np.int64):
        for e in range(ppb):
            ok = ppb == 1 or j * kv_block + e * (kv_block // ppb) < L
            out.append(int(page_table_row[j * ppb + e]) if ok else -1)
    return np.asarray(out, dtype=np.int64)


def check_kap_row(gpu_blocks, gpu_pages, gpu_count, gpu_hrm_count, tile: TileProxy,
                  page_table_row, w_rtol=W_RTOL, gap=HRM_GAP, ppb=1, kv_block=None,
                  L=None) -> str:
    """'exact' if the row equals the oracle's, 'tie' if it differs only where
    the oracle's own scores are within the near-tie tolerances; raises
    AssertionError otherwise.  ``gpu_pages`` holds ppb pages per slot."""
    k = tile.k
    C = len(gpu_blocks)
    assert int(gpu_count) == k, f"count {gpu_count} != {k}"
    g = np.asarray(gpu_blocks[:k], dtype=np.int64)
    assert np.all(np.asarray(gpu_blocks[k:]) == -1), "slots past the count must be -1"
    assert np.all(np.asarray(gpu_pages[k * ppb:]) == -1), "pages past the count must be -1"
    assert np.array_equal(np.asarray(gpu_pages[:k * ppb]),
                          expected_pages(g, page_table_row, ppb, kv_block, L)), "page remap mismatch"
    assert C >= k
    if np.array_equal(g, tile.blocks) and int(gpu_hrm_count) == tile.hrm_count:
        return "exact"
    # --- every difference must be explained by near-ties of the oracle's scores
    n = tile.n
    assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < n, "not a candidate subset"
    certain, possible = _hrm_sets(tile, gap)
    hc = int(gpu_hrm_count)
    assert 0 <= hc <= k
    gh, gn = g[:hc], g[hc:]
    assert set(gh.tolist()) <= possible, f"GPU HRM blocks {set(gh.tolist()) - possible} not near a row max"
    assert not (set(gn.tolist()) & certain), "a certain HRM block sits in the non-HRM group"
    w = tile.w

    def close(a, b):
        return abs(w[a] - w[b]) <= w_rtol * max(w[a], w[b]) + 1e-12

    for grp in (gh, gn):
        for a, b in zip(grp, grp[1:]):
            assert w[a] >= w[b] or close(a, b), f"order inversion {a},{b}: {w[a]} < {w[b]}"
    unsel = set(range(n)) - set(g.tolist())
    if hc < k:   # the whole HRM group was kept, then the best non-HRM blocks
        assert not (unsel & certain), "a certain HRM block was dropped"
        if len(gn):
            worst = gn[np.argmin(w[gn])]
            for u in unsel:
                assert w[u] <= w[worst] or close(u, worst), f"dropped block {u} beats kept {worst}"
    else:        # only HRM blocks kept
        if len(gh):
            worst = gh[np.argmin(w[gh])]
            for u in unsel & certain:
                assert w[u] <= w[worst] or close(u, worst), f"dropped HRM {u} beats kept {worst}"
    return "tie"


# ---------------------------------------------------------------------------
# OSK tiles


def check_osk_tile(gpu_out_rows, gpu_lse_rows, gpu_skip, res, q_rows, row_pos, k, v, blocks,
                   scale, kv_block, stats: ErrStats, lse_stats: ErrStats,
                   margin_tol=MARGIN_TOL, max_variants=16) -> int:
    """Compare one tile; returns the number of near-threshold slots.

    ``res`` is the oracle's TileResult for the same visited list.  Slots whose
    oracle margin is within ``margin_tol`` of the threshold may be decided
    either way; the oracle recomputes the output for every combination of
    those decisions and the GPU output must match the combination its skip
    record names, which must agree with the oracle on every other slot.
    """
    gpu_skip = np.asarray(gpu_skip[:len(blocks)], dtype=bool)
    near = np.flatnonzero(np.abs(res.margin) < margin_tol)
    firm = np.setdiff1d(np.arange(len(blocks)), near)
    assert np.array_equal(gpu_skip[firm], res.skipped[firm]), (
        f"skip decisions differ at firm slots {firm[gpu_skip[firm] != res.skipped[firm]]}")
    ref_out, ref_lse = res.out, res.lse
    if len(near):
        assert 2 ** len(near) <= max_variants, "too many near-threshold slots in one tile"
        L = k.shape[0]
        best = None
        for combo in itertools.product([False, True], repeat=len(near)):
            dec = res.skipped.copy()
            dec[near] = combo
            key_ok = np.zeros(L, dtype=bool)
            for j, sk in zip(blocks, dec):
                if not sk:
                    key_ok[j * kv_block:min((j + 1) * kv_block, L)] = True
            o, ls = odense.attention_rows(q_rows, row_pos, k, v, scale, key_ok=key_ok)
            if np.array_equal(dec, gpu_skip):
                best = (o, ls)
        assert best is not None, "GPU skip record is not one of the allowed variants"
        ref_out, ref_lse = best
    stats.add(np.asarray(gpu_out_rows), ref_out)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gpu_lse_rows), fin), "rows without keys disagree"
    lse_stats.add(np.asarray(gpu_lse_rows)[fin], ref_lse[fin])
    return len(near)
