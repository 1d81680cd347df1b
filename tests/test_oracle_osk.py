"""Pins for the Ordered-Skipping Kernel oracle (CPU, float64).

* budget 100% with the skip off (Delta = -1, CoSA (paperpeel) App. D.1) in
  ascending order reproduces dense causal attention;
* order invariance of the online softmax (§3.2 P2, §4.3 "Any-order page
  visiting"): any visiting order of a fixed visited set gives the same output;
* the sequential loop and the closed form (prefix-max) agree exactly on the
  skip set and to rounding on the output;
* the output equals torch SDPA (float64, CPU) with an explicit mask over the
  computed keys (library routine);
* hand-worked examples of the skip rule, its direction, the first-block rule
  and the per-row AND ("bucket effect", §3.3 L2.2);
* tau monotonicity and the three-way block partition (§4.1, Figure 4 text).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import cosa_inputs as ci
from oracle import dense, kap, osk
from oracle.paging import materialise


def _inputs(name, **kw):
    w = ci.get(name)
    if kw:
        w = w.with_(**kw)
    return w, ci.make(w).bf16_rounded()


def test_full_budget_no_skip_equals_dense_ragged():
    w, x = _inputs("tiny", seqlens=(300, 1, 129, 64), num_q_heads=4, num_kv_heads=2,
                   shuffled_pages=True, spare_pages=5)
    blocks, counts = osk.dense_order_mask(x.cu_seqlens, 4, 64, 64)
    r = osk.osk_prefill(x.q, x.k_pool, x.v_pool, x.page_table, x.cu_seqlens, 2, 64, 64,
                        blocks, counts, -1.0, w.softmax_scale)
    for b, s, L in [(b, int(x.cu_seqlens[b]), int(x.seqlens[b])) for b in range(4)]:
        k = materialise(x.k_pool, x.page_table[b], L, 64)
        v = materialise(x.v_pool, x.page_table[b], L, 64)
        out, lse = dense.dense_causal_attention(x.q[s:s + L].astype(np.float64), k, v,
                                                w.softmax_scale)
        assert np.max(np.abs(r.out[s:s + L] - out)) < 1e-12
        assert np.max(np.abs(r.lse[:, s:s + L] - lse)) < 1e-12
    assert np.all(r.skip_record == 0)
    assert np.all(np.isfinite(r.out))


def test_full_budget_kap_order_no_skip_equals_dense():
    # the KAP order at budget 100% is a permutation of all candidates
    w, x = _inputs("tiny", seqlens=(640,))
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, 2, 64, 64, 1.0,
                               w.softmax_scale)
    r = osk.osk_prefill(x.q, x.k_pool, x.v_pool, x.page_table, x.cu_seqlens, 2, 64, 64,
                        m.blocks, m.counts, -1.0, w.softmax_scale)
    k = materialise(x.k_pool, x.page_table[0], 640, 64)
    v = materialise(x.v_pool, x.page_table[0], 640, 64)
    out, _ = dense.dense_causal_attention(x.q.astype(np.float64), k, v, w.softmax_scale)
    assert np.max(np.abs(r.out - out)) < 1e-12


def _tile_args(x, w, h, i, L=None):
    L = int(x.seqlens[0]) if L is None else L
    g = h // (w.num_q_heads // w.num_kv_heads)
    k = materialise(x.k_pool, x.page_table[0], L, 64)[:, g]
    v = materialise(x.v_pool, x.page_table[0], L, 64)[:, g]
    rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
    return x.q[rows, h].astype(np.float64), rows, k, v


def test_order_invariance_without_skip():
    w, x = _inputs("tiny")
    rng = np.random.default_rng(0)
    for h, i in [(0, 31), (1, 17), (0, 0)]:
        qr, rows, k, v = _tile_args(x, w, h, i)
        blocks = list(range(i + 1))
        base = osk.osk_tile_sequential(qr, rows, k, v, blocks, -1.0, w.softmax_scale, 64)
        for _ in range(3):
            perm = list(rng.permutation(blocks))
            r = osk.osk_tile_sequential(qr, rows, k, v, perm, -1.0, w.softmax_scale, 64)
            assert np.max(np.abs(r.out - base.out)) < 1e-12
            assert np.max(np.abs(r.lse - base.lse)) < 1e-12


@pytest.mark.parametrize("tau", [0.0, 2.0, 8.0, 12.0])
def test_sequential_equals_closed_form_and_sdpa(tau):
    w, x = _inputs("tiny_skip")
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, 2, 64, 64, 0.5,
                               w.softmax_scale)
    n_skipped = 0
    for h in range(2):
        for i in range(0, 32, 3):
            qr, rows, k, v = _tile_args(x, w, h, i)
            blocks = m.blocks[0, h, i, :m.counts[0, h, i]]
            a = osk.osk_tile_sequential(qr, rows, k, v, blocks, tau, w.softmax_scale, 64)
            b = osk.osk_tile_closed_form(qr, rows, k, v, blocks, tau, w.softmax_scale, 64)
            assert np.array_equal(a.skipped, b.skipped)
            assert np.array_equal(a.margin, b.margin)
            assert np.array_equal(a.skipped, a.margin < 0)
            assert np.max(np.abs(a.out - b.out)) < 1e-12
            assert np.max(np.abs(a.lse - b.lse)) < 1e-12
            n_skipped += int(a.skipped.sum())
            # SDPA over exactly the computed keys
            L = k.shape[0]
            allowed = np.zeros((len(rows), L), dtype=bool)
            for j, sk in zip(blocks, a.skipped):
                if not sk:
                    allowed[:, j * 64:(j + 1) * 64] = True
            allowed &= np.arange(L)[None, :] <= rows[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qr)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
                attn_mask=torch.from_numpy(allowed)[None], scale=w.softmax_scale)[0].numpy()
            assert np.max(np.abs(a.out - ref)) < 1e-12
    if tau <= 8.0:
        assert n_skipped > 0, "the skip-variant input should make the skip fire"


def test_skip_rule_hand_example():
    # one query row at position 3, two key blocks of two keys, scale 1, D = 1.
    # block 0 logits (10, 10), block 1 logits (0, 0).
    q = np.array([[1.0]])
    pos = np.array([3])
    k = np.array([[10.0], [10.0], [0.0], [0.0]])
    v = np.array([[1.0], [3.0], [5.0], [7.0]])
    e10 = math.exp(10.0)
    full = (e10 * 1 + e10 * 3 + 5 + 7) / (2 * e10 + 2)
    # order [0, 1], tau = 8: after block 0, m = 10; block 1 max 0 < 10 - 8 -> skipped.
    r = osk.osk_tile_sequential(q, pos, k, v, [0, 1], 8.0, 1.0, 2)
    assert list(r.skipped) == [False, True]
    assert abs(r.out[0, 0] - 2.0) < 1e-15               # mean of v0, v1
    assert abs(r.margin[1] - (0 - 10 + 8)) < 1e-15
    assert abs(r.lse[0] - (10 + math.log(2))) < 1e-15
    # tau = 12: 0 < -2 is false -> computed, full softmax
    r = osk.osk_tile_sequential(q, pos, k, v, [0, 1], 12.0, 1.0, 2)
    assert list(r.skipped) == [False, False]
    assert abs(r.out[0, 0] - full) < 1e-15
    # order [1, 0]: the first block is never skipped (m = -inf); block 0 then
    # raises the max, it is not negligible -> nothing skipped, same result
    r = osk.osk_tile_sequential(q, pos, k, v, [1, 0], 8.0, 1.0, 2)
    assert list(r.skipped) == [False, False]
    assert abs(r.out[0, 0] - full) < 1e-13
    # tau < 0 switches the skip off
    r = osk.osk_tile_sequential(q, pos, k, v, [0, 1], -1.0, 1.0, 2)
    assert list(r.skipped) == [False, False]


def test_bucket_effect_one_row_vetoes():
    # two rows; block 1 is negligible for row 0 but not for row 1
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    pos = np.array([3, 3])
    k = np.array([[10.0, 0.0], [10.0, 0.0], [0.0, 0.0], [0.0, 0.0]])
    v = np.arange(4.0)[:, None]
    r = osk.osk_tile_sequential(q, pos, k, v, [0, 1], 8.0, 1.0, 2)
    # row 1 sees logits 0 everywhere: m = 0 after block 0, block 1 max 0 is not
    # below 0 - 8, so row 1 vetoes the skip even though row 0 agrees
    assert list(r.skipped) == [False, False]
    assert abs(r.out[1, 0] - 1.5) < 1e-15                # uniform over 4 keys
    # drop row 1: now the tile skips block 1
    r = osk.osk_tile_sequential(q[:1], pos[:1], k, v, [0, 1], 8.0, 1.0, 2)
    assert list(r.skipped) == [False, True]


def test_tau_monotone_and_partition():
    w, x = _inputs("tiny_skip")
    m = kap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, 2, 64, 64, 0.5,
                               w.softmax_scale)
    prev = None
    for tau in [1.0, 4.0, 8.0, 16.0]:
        r = osk.osk_prefill(x.q, x.k_pool, x.v_pool, x.page_table, x.cu_seqlens, 2, 64, 64,
                            m.blocks, m.counts, tau, w.softmax_scale, closed_form=True)
        cur = r.skip_record.astype(bool)
        if prev is not None:
            assert np.all(cur <= prev)       # larger tau -> subset of skipped slots
        prev = cur
        # partition: mask-skipped + in-kernel skipped + computed = candidates
        for h in range(2):
            for i in range(32):
                n = i + 1
                visited, skipped = r.row_stats[0, h, i]
                computed = visited - skipped
                assert (n - visited) + skipped + computed == n
                assert visited == m.counts[0, h, i]


# ---------------------------------------------------------------------------
# Length-adaptive threshold Delta / N (CoSA (paperpeel) §5.1, App. D.1)


def test_tau_from_delta_hand_values():
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "kap_worked_examples.json")) as f:
        cases = json.load(f)["delta_threshold"]["cases"]
    for n, delta, tau in cases:
        assert abs(osk.tau_from_delta(n, delta) - tau) < 1e-6


def _two_block_sequence():
    """L = 4, page 2, D = 1, q = 1, keys (1, 1 | 0.5, 0.5), values (1, 1 | 3, 3),
    identity pages, one 4-row tile visiting [0, 1]."""
    q = np.ones((4, 1, 1))
    k_pool = np.array([1.0, 1.0, 0.5, 0.5]).reshape(2, 1, 2, 1)
    v_pool = np.array([1.0, 1.0, 3.0, 3.0]).reshape(2, 1, 2, 1)
    pt = np.array([[0, 1]])
    cu = np.array([0, 4])
    blocks = np.array([0, 1], dtype=np.int32).reshape(1, 1, 1, 2)
    counts = np.array([2], dtype=np.int32).reshape(1, 1, 1)
    return q, k_pool, v_pool, pt, cu, blocks, counts


@pytest.mark.parametrize("closed", [False, True])
def test_delta_mode_negative_tau_still_skips(closed):
    """With N = 4 and Delta = 4e, tau = ln(N / Delta) = -1 < 0: in the Delta / N
    mode the skip stays on.  After block 0 every row has m = 1; block 1 has
    bm = 0.5 for rows 2-3 (0.5 < 1 + 1) and -inf for rows 0-1, so the tile
    skips it and rows 2-3 average block 0's values only (out = 1).  With the
    plain tau = -1 (skip off) row 2 (keys 0-2) gets (2e*1 + e^0.5*3) / (2e + e^0.5)
    and row 3 (keys 0-3) gets (2e*1 + 2e^0.5*3) / (2e + 2e^0.5)."""
    q, kp, vp, pt, cu, blocks, counts = _two_block_sequence()
    on = osk.osk_prefill(q, kp, vp, pt, cu, 1, 4, 2, blocks, counts, tau=0.0, scale=1.0,
                         closed_form=closed, delta=4 * math.e)
    assert on.skip_record[0, 0, 0].tolist() == [0, 1]
    assert np.allclose(on.out[:, 0, 0], 1.0, atol=1e-15)
    off = osk.osk_prefill(q, kp, vp, pt, cu, 1, 4, 2, blocks, counts, tau=-1.0, scale=1.0,
                          closed_form=closed)
    assert off.skip_record[0, 0, 0].tolist() == [0, 0]
    e, h = math.e, math.exp(0.5)
    want = [(2 * e + h * 3) / (2 * e + h), (2 * e + 2 * h * 3) / (2 * e + 2 * h)]
    assert np.allclose(off.out[2:, 0, 0], want, atol=1e-14)
    assert np.allclose(off.out[:2, 0, 0], 1.0, atol=1e-15)
    # Delta <= 0 switches the skip off in the Delta / N mode as well
    neg = osk.osk_prefill(q, kp, vp, pt, cu, 1, 4, 2, blocks, counts, tau=5.0, scale=1.0,
                          closed_form=closed, delta=-1.0)
    assert neg.skip_record[0, 0, 0].tolist() == [0, 0]
    # tau_b = ln(4 / Delta) = 0.6 > bm-margin: 0.5 < 1 - 0.6 is false, computed
    mid = osk.osk_prefill(q, kp, vp, pt, cu, 1, 4, 2, blocks, counts, tau=0.0, scale=1.0,
                          closed_form=closed, delta=4 * math.exp(-0.6))
    assert mid.skip_record[0, 0, 0].tolist() == [0, 0]
    lo = osk.osk_prefill(q, kp, vp, pt, cu, 1, 4, 2, blocks, counts, tau=0.0, scale=1.0,
                         closed_form=closed, delta=4 * math.exp(-0.4))
    assert lo.skip_record[0, 0, 0].tolist() == [0, 1]
