"""Pins and a CPU report for the proxy-fidelity analysis (oracle/fidelity.py).

The exact block mass is pinned to a hand-derived uniform-attention case and
to brute force; the report computes IoU of the KAP kept set against the exact
top-k blocks at matched budgets on a llama-shaped synthetic sequence (the
analogue of the proxy-fidelity figure of CoSA (paperpeel) §3.2, Fig. 2) and
checks what holds by construction: the exact top-k set covers at least the
proxy's mass, and a 100% budget gives IoU 1.
"""
import math

import numpy as np

import cosa_inputs as ci
from oracle import fidelity
from oracle.paging import materialise


def test_uniform_attention_block_mass_by_hand():
    # q = 0: row t attends uniformly to keys 0..t.  Tile rows 4..7, blocks of
    # 4 keys: block 0 gets 4/(t+1) of row t, block 1 the rest.
    k = np.random.default_rng(0).standard_normal((8, 3))
    rows = np.arange(4, 8)
    m = fidelity.exact_block_mass(np.zeros((4, 3)), rows, k, 0.7, 4)
    b0 = (4 / 5 + 4 / 6 + 4 / 7 + 4 / 8) / 4
    assert np.allclose(m, [b0, 1 - b0], atol=1e-15)


def test_block_mass_brute_force():
    rng = np.random.default_rng(1)
    L, D, kb = 23, 4, 5
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    rows = np.arange(10, 23)
    got = fidelity.exact_block_mass(q[rows], rows, k, 0.9, kb)
    want = np.zeros(len(got))
    for t in rows:
        w = [math.exp(0.9 * sum(q[t, d] * k[u, d] for d in range(D))) for u in range(t + 1)]
        z = math.fsum(w)
        for u in range(t + 1):
            want[u // kb] += w[u] / z / len(rows)
    assert np.allclose(got, want, atol=1e-13)
    assert abs(got.sum() - 1.0) < 1e-13


def test_top_mass_and_iou_hand_values():
    assert list(fidelity.top_mass_blocks(np.array([0.1, 0.4, 0.4, 0.1]), 2)) == [1, 2]
    assert list(fidelity.top_mass_blocks(np.array([0.25, 0.25, 0.5]), 2)) == [2, 0]
    assert fidelity.iou([0, 1, 2], [1, 2, 3]) == 0.5
    assert fidelity.iou([], []) == 1.0
    assert fidelity.iou([4], [5]) == 0.0


def test_proxy_fidelity_report():
    w = ci.get("llama32k").with_(seqlens=(8192,), num_q_heads=4, num_kv_heads=1)
    x = ci.make(w).bf16_rounded()
    L = int(x.cu_seqlens[1])
    keys = materialise(x.k_pool, x.page_table[0], L, w.page_size)[:, 0, :].astype(np.float64)
    budgets = (1.0, 0.5, 0.3, 0.2, 0.1, 0.05)
    tiles = list(range(8, 64, 4))
    rows = {b: [] for b in budgets}
    for h in range(w.num_q_heads):
        for r in fidelity.proxy_fidelity(x.q[:L, h].astype(np.float64), keys, w.softmax_scale,
                                         w.q_block, w.page_size, budgets, tiles=tiles):
            rows[r.budget].append(r)
            assert r.oracle_mass >= r.proxy_mass - 1e-12
            assert 0.0 <= r.mean_iou <= 1.0
            if r.budget == 1.0:
                assert r.mean_iou == 1.0
    print("\n[fidelity] llama-shaped 8K, 4 heads, 14 tiles/head: budget, IoU, proxy mass, "
          "top-k mass")
    for b in budgets:
        rs = rows[b]
        print(f"[fidelity] {b:5.2f} {np.mean([r.mean_iou for r in rs]):.3f} "
              f"{np.mean([r.proxy_mass for r in rs]):.3f} "
              f"{np.mean([r.oracle_mass for r in rs]):.3f}")
