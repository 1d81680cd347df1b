"""Pins for the Kernel-Aware Proxy oracle (CPU, float64).

* hand-derived golden cases (tests/golden/kap_worked_examples.json) for the
  flag-grouped order, HRM-first truncation and tie-breaks (CoSA (paperpeel)
  App. C.1 and §4.2 "Flag-grouped sorting");
* the pooled-score identity: the pooled logit equals the mean of the exact
  logits over the (proxy row x key block) sub-block, by brute force;
* the structural invariants of M_KAP the pages state: a subset of the causal
  candidates, HRM group before the non-HRM group, each group sorted by score,
  length equal to the budget count (§4.1, App. C.1);
* budget 100% keeps every candidate.
"""
import json
import math
import os

import numpy as np
import pytest

import cosa_inputs as ci
from oracle import kap
from oracle.paging import materialise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kap_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _example_arrays(ex):
    L, g, kb, D = ex["L"], ex["rows_per_proxy"], ex["kv_block"], ex["D"]
    q = np.zeros((L, D))
    for r, vec in enumerate(ex["proxy_row_query"]):
        q[r * g:(r + 1) * g] = vec
    k = np.zeros((L, D))
    for j, vec in enumerate(ex["block_key"]):
        k[j * kb:(j + 1) * kb] = vec
    return q, k


@pytest.mark.parametrize("idx", [0, 1])
def test_golden_worked_example(idx):
    ex = _golden()["examples"][idx]
    q, k = _example_arrays(ex)
    res = kap.head_tiles(q, k, ex["scale"], ex["q_block"], ex["kv_block"],
                         kap.budget_ppm(ex["budget"]), ex["rows_per_proxy"])
    assert list(res) == [0]
    t = res[0]
    assert t.n == ex["expect_n"]
    assert np.allclose(t.w, ex["expect_w"], rtol=0, atol=1e-15)
    assert list(t.hrm) == ex["expect_hrm"]
    assert list(t.order) == ex["expect_order"]
    assert t.k == ex["expect_k"]
    assert list(t.blocks) == ex["expect_blocks"]
    assert t.hrm_count == ex["expect_hrm_count"]


def test_budget_counts_hand_values():
    for n, beta, want in _golden()["budget_counts"]["cases"]:
        assert kap.budget_count(n, kap.budget_ppm(beta)) == want, (n, beta)
    assert kap.budget_count(0, 100000) == 0
    with pytest.raises(ValueError):
        kap.budget_ppm(0.0)
    with pytest.raises(ValueError):
        kap.budget_ppm(1.5)


def test_pooled_score_equals_mean_of_exact_logits():
    rng = np.random.default_rng(3)
    L, D, qb, kb, g = 77, 5, 32, 8, 16
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    scale = 0.37
    kbar = kap.pooled_keys(k, kb)
    qbar, last, valid = kap.pooled_queries(q, qb, g)
    for i in range(qbar.shape[0]):
        for r in range(qbar.shape[1]):
            rows = [t for t in range(i * qb + r * g, i * qb + (r + 1) * g) if t < L]
            assert valid[i, r] == bool(rows)
            if not rows:
                continue
            assert last[i, r] == rows[-1]
            for j in range(kbar.shape[0]):
                keys = [u for u in range(j * kb, (j + 1) * kb) if u < L]
                brute = sum(scale * float(q[a] @ k[u]) for a in rows for u in keys)
                brute /= len(rows) * len(keys)
                assert abs(scale * float(qbar[i, r] @ kbar[j]) - brute) < 1e-13


def _check_tile_invariants(t: kap.TileProxy, last_rows, kv_block):
    n = t.n
    assert n == int(max(last_rows)) // kv_block + 1
    order = list(t.order)
    assert sorted(order) == list(range(n))                    # a permutation
    blocks = list(t.blocks)
    assert len(blocks) == t.k and len(set(blocks)) == len(blocks)
    flags = [bool(t.hrm[j]) for j in order]
    # every HRM block precedes every non-HRM block
    assert flags == sorted(flags, reverse=True)
    # each group sorted by w desc, then block index asc
    for a, b in zip(order, order[1:]):
        if t.hrm[a] == t.hrm[b]:
            assert (t.w[a] > t.w[b]) or (t.w[a] == t.w[b] and a < b)
    # HRM flags: exactly the arg-max blocks of the proxy rows
    am = set(int(np.argmax(row)) for row in t.scores)
    assert set(np.flatnonzero(t.hrm).tolist()) == am
    # probabilities: each proxy row sums to 1 over its candidates only
    for r, lr in enumerate(last_rows):
        c = int(lr) // kv_block + 1
        assert abs(t.probs[r, :c].sum() - 1) < 1e-12
        assert np.all(t.probs[r, c:] == 0)
    assert abs(t.w.sum() - 1) < 1e-12


@pytest.mark.parametrize("name", ["tiny", "tiny_skip"])
def test_tiny_mask_invariants(name):
    w = ci.get(name)
    x = ci.make(w).bf16_rounded()
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                               w.q_block, w.page_size, w.budget, w.softmax_scale)
    L = w.seqlens[0]
    nqb = (L + w.q_block - 1) // w.q_block
    assert m.capacity == kap.budget_count((L + 63) // 64, kap.budget_ppm(w.budget))
    for h in range(w.num_q_heads):
        for i in range(nqb):
            t = m.tiles[(0, h, i)]
            last_rows = [min(i * w.q_block + (r + 1) * 16, L) - 1
                         for r in range(w.q_block // 16) if i * w.q_block + r * 16 < L]
            _check_tile_invariants(t, last_rows, w.page_size)
            cnt = m.counts[0, h, i]
            assert cnt == kap.budget_count(i + 1, kap.budget_ppm(w.budget))
            assert np.array_equal(m.blocks[0, h, i, :cnt], t.blocks)
            assert np.all(m.blocks[0, h, i, cnt:] == -1)
            assert np.array_equal(m.pages[0, h, i, :cnt], x.page_table[0][t.blocks])
            assert m.hrm_counts[0, h, i] == t.hrm_count


def test_budget_full_selects_every_candidate_ragged_batch():
    w = ci.get("tiny").with_(seqlens=(200, 64, 1, 130), num_q_heads=4, num_kv_heads=2,
                              shuffled_pages=True, spare_pages=3)
    x = ci.make(w).bf16_rounded()
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, 2, 64, 64,
                               1.0, w.softmax_scale)
    for b, L in enumerate(w.seqlens):
        for h in range(4):
            for i in range((L + 63) // 64):
                n = (min((i + 1) * 64, L) - 1) // 64 + 1
                assert m.counts[b, h, i] == n
                assert sorted(m.blocks[b, h, i, :n].tolist()) == list(range(n))
            assert np.all(m.counts[b, h, (L + 63) // 64:] == 0)


def test_kap_independent_of_page_placement():
    # the same logical keys stored under two different page permutations give
    # the same mask, and pages follow each table
    w = ci.get("tiny").with_(seqlens=(300,), shuffled_pages=False, spare_pages=0)
    x = ci.make(w).bf16_rounded()
    perm = np.array([3, 0, 4, 1, 2])
    kp = np.empty_like(x.k_pool)
    kp[perm] = x.k_pool[x.page_table[0, :5]]
    pt = perm[None, :].astype(np.int32)
    a = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, 2, 64, 64, 0.5, 0.125)
    b = kap.proxy_ordered_mask(x.q, kp, pt, x.cu_seqlens, 2, 64, 64, 0.5, 0.125)
    assert np.array_equal(a.blocks, b.blocks)
    assert np.array_equal(b.pages[b.blocks >= 0], perm[b.blocks[b.blocks >= 0]])
    assert np.allclose(materialise(kp, pt[0], 300, 64), materialise(x.k_pool, x.page_table[0], 300, 64))


# ---------------------------------------------------------------------------
# Stage-1 Top-p (CoSA (paperpeel) §5.1 "Hyperparameters", App. D.1)


@pytest.mark.parametrize("case", range(9))
def test_top_p_golden(case):
    g = _golden()
    ex_idx, p, cap, want_k, want_blocks = g["top_p"]["cases"][case]
    ex = g["examples"][ex_idx]
    q, k = _example_arrays(ex)
    res = kap.head_tiles(q, k, ex["scale"], ex["q_block"], ex["kv_block"], kap.budget_ppm(cap),
                         ex["rows_per_proxy"], top_p=p)
    t = res[0]
    assert t.k == want_k
    assert list(t.blocks) == want_blocks


def test_top_p_count_hand_values():
    for w, p, want in _golden()["top_p"]["count_cases"]:
        assert kap.top_p_count(np.asarray(w), p) == want, (w, p)
    assert kap.top_p_count(np.zeros(0), 0.5) == 0
    for bad in (0.0, -0.1, 1.5):
        with pytest.raises(ValueError):
            kap.top_p_count(np.ones(3) / 3, bad)


def test_top_p_invariants_on_random_tiles():
    """Kept mass reaches p and the kept prefix minus its last block does not;
    the count grows with p; p = 1 keeps every candidate."""
    x = ci.make(ci.get("tiny"))
    w_ = x.workload
    L = int(x.cu_seqlens[1])
    keys = materialise(x.k_pool, x.page_table[0], L, w_.page_size)
    for h in range(w_.num_q_heads):
        g = h // (w_.num_q_heads // w_.num_kv_heads)
        prev = None
        for p in (0.3, 0.6, 0.9, 0.95, 1.0):
            tiles = kap.head_tiles(x.q[:L, h, :].astype(np.float64), keys[:, g, :].astype(np.float64),
                                   w_.softmax_scale, w_.q_block, w_.page_size, kap.budget_ppm(1.0),
                                   top_p=p)
            ks = np.array([t.k for t in tiles.values()])
            for t in tiles.values():
                mass = math.fsum(t.w[t.order[:t.k]])
                if p < 1.0:
                    assert mass >= p and math.fsum(t.w[t.order[:t.k - 1]]) < p
                else:
                    assert t.k == t.n
                assert abs(math.fsum(t.w) - 1.0) < 1e-12
            if prev is not None:
                assert np.all(ks >= prev)
            prev = ks


# ---------------------------------------------------------------------------
# KV-group-shared masks (one mask per KV head for its query heads)


def test_gqa_shared_golden():
    ex = _golden()["gqa_shared"]
    L, kb = ex["L"], ex["kv_block"]
    k = np.zeros((L, ex["D"]))
    for j, vec in enumerate(ex["block_key"]):
        k[j * kb:(j + 1) * kb] = vec
    qs = [np.tile(np.asarray(v, dtype=np.float64), (L, 1)) for v in ex["head_query"]]
    beta = kap.budget_ppm(ex["budget"])
    t = kap.group_tiles(qs, k, ex["scale"], ex["q_block"], kb, beta, ex["rows_per_proxy"])[0]
    assert np.allclose(t.w, ex["expect_w"], rtol=0, atol=1e-15)
    assert list(t.hrm) == ex["expect_hrm"]
    assert list(t.order) == ex["expect_order"]
    assert list(t.blocks) == ex["expect_blocks"]
    for qh, want in zip(qs, ex["expect_per_head_blocks"]):
        alone = kap.head_tiles(qh, k, ex["scale"], ex["q_block"], kb, beta, ex["rows_per_proxy"])[0]
        assert list(alone.blocks) == want


def test_gqa_shared_brute_force_importance():
    """w_j of the shared mask is the mean over every head's proxy rows of that
    row's softmax over its own candidates, written out with loops."""
    rng = np.random.default_rng(7)
    L, D, qb, kb, g = 150, 3, 64, 16, 16
    qs = [rng.standard_normal((L, D)) for _ in range(3)]
    k = rng.standard_normal((L, D))
    scale = 0.6
    res = kap.group_tiles(qs, k, scale, qb, kb, kap.budget_ppm(1.0), g)
    for i, t in res.items():
        rows = []
        for qh in qs:
            for r in range(qb // g):
                pos = [x for x in range(i * qb + r * g, i * qb + (r + 1) * g) if x < L]
                if not pos:
                    continue
                qbar = [sum(qh[x, d] for x in pos) / len(pos) for d in range(D)]
                cand = pos[-1] // kb + 1
                kbar = [[sum(k[u, d] for u in range(j * kb, min((j + 1) * kb, L))) /
                         (min((j + 1) * kb, L) - j * kb) for d in range(D)] for j in range(cand)]
                sc = [scale * sum(qbar[d] * kbar[j][d] for d in range(D)) for j in range(cand)]
                mx = max(sc)
                z = math.fsum(math.exp(v - mx) for v in sc)
                rows.append([math.exp(v - mx) / z for v in sc] + [0.0] * (t.n - cand))
        w = np.mean(np.asarray(rows), axis=0)
        assert np.allclose(t.w, w, atol=1e-12)


def test_gqa_shared_equals_per_head_for_one_head_groups():
    x = ci.make(ci.get("tiny"))
    w_ = x.workload
    a = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w_.num_kv_heads,
                               w_.q_block, w_.page_size, w_.budget, w_.softmax_scale)
    b = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w_.num_kv_heads,
                               w_.q_block, w_.page_size, w_.budget, w_.softmax_scale,
                               shared_kv=True)
    assert w_.num_q_heads == w_.num_kv_heads
    for f in ("blocks", "pages", "counts", "hrm_counts"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_two_page_logical_blocks_remap_pages():
    """kv_block = 2 pages: every kept block lists its two pages (page table
    entries 2j, 2j+1), and -1 for a second page past the sequence's end."""
    w = ci.get("tiny").with_(seqlens=(129, 200, 64), kv_block=128, shuffled_pages=True,
                             spare_pages=3)
    x = ci.make(w)
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                               w.q_block, 128, 1.0, w.softmax_scale)
    assert m.pages.shape[-1] == 2 * m.blocks.shape[-1]
    for b, L in enumerate(w.seqlens):
        for idx in np.ndindex(*m.counts.shape[1:]):
            c = m.counts[(b,) + idx]
            for t in range(c):
                j = m.blocks[(b,) + idx][t]
                p0, p1 = m.pages[(b,) + idx][2 * t:2 * t + 2]
                assert p0 == x.page_table[b][2 * j]
                assert p1 == (x.page_table[b][2 * j + 1] if 128 * j + 64 < L else -1)
            assert np.all(m.pages[(b,) + idx][2 * c:] == -1)
