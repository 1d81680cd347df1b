"""GPU parity: every kernel through the C ABI against the CPU fp64 oracle.

Inputs are seeded synthetic workloads (cosa_inputs), rounded to bf16 once;
the GPU gets the bf16 tensors, the oracle the same values widened to fp64.
Tolerances: max-abs 2e-2 / mean-abs 2e-3 on outputs for the same visited set;
masks and page remaps bit-exact except near-ties of the oracle's own scores;
skip sets identical except slots within 1e-3 nats of the threshold (counted).
"""
import dataclasses

import numpy as np
import pytest

import block_sparse_long_kap_amd as bk
import cosa_inputs as ci
from oracle import dense as odense
from oracle import kap as okap
from oracle import osk as oosk
from oracle.paging import materialise

from .parity import (ErrStats, check_kap_row, check_osk_tile, expected_pages, report,
                     selection_on_own_scores, upload)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(name, **kw):
    w = ci.get(name)
    if kw:
        w = w.with_(**kw)
    return w, ci.make(w).bf16_rounded()


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _dense_oracle(x, w):
    out = np.zeros(x.q.shape)
    lse = np.full((w.num_q_heads, x.q.shape[0]), -np.inf)
    for b in range(w.batch):
        s, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        if L == 0:
            continue
        k = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        v = materialise(x.v_pool, x.page_table[b], L, w.page_size)
        o, ls = odense.dense_causal_attention(x.q[s:s + L].astype(np.float64), k, v,
                                              w.softmax_scale)
        out[s:s + L] = o
        lse[:, s:s + L] = ls
    return out, lse


RAGGED = dict(seqlens=(1, 63, 64, 65, 200, 383), num_q_heads=8, num_kv_heads=2,
              head_dim=128, q_block=128, shuffled_pages=True, spare_pages=7,
              precision="bf16")


@pytest.mark.parametrize("case", [
    ("tiny", {}),
    ("tiny", dict(RAGGED)),
    ("tiny", dict(RAGGED, q_block=64)),
    ("tiny", dict(RAGGED, head_dim=64, q_block=128)),
    # query heads per KV group 3 (one head per workgroup), 1 and 2 (two), and
    # longer sequences: whole groups of four pipeline stages plus remainders
    ("tiny", dict(RAGGED, num_q_heads=6, num_kv_heads=2)),
    ("tiny", dict(RAGGED, num_q_heads=4, num_kv_heads=4)),
    ("tiny", dict(RAGGED, num_q_heads=4, num_kv_heads=2, seqlens=(700, 1031, 129))),
])
def test_dense_matches_oracle(case):
    name, kw = case
    w, x = _inputs(name, **kw)
    print(f"[case] dense {name} {kw}", flush=True)
    prob, q, k, v = upload(x, DEV)
    res = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    ref, ref_lse = _dense_oracle(x, w)
    st, ls = ErrStats(), ErrStats()
    st.add(_np(res.out), ref)
    ls.add(_np(res.lse), ref_lse)
    st.assert_ok(label=f"dense {name} out")
    ls.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"dense {name} lse")


def _run_osk_vs_oracle(w, x, blocks, counts, tau, label, tiles=None, delta=None,
                       shared=False):
    """OSK through the C ABI against the closed-form oracle tile by tile; with
    ``delta`` the length-adaptive entry point and tau_b = ln(L_b / delta); with
    ``shared`` the masks are per KV head (cosa_osk_prefill_shared_kv)."""
    prob, q, k, v = upload(x, DEV)
    C = blocks.shape[-1]
    ppb = w.block // w.page_size
    pages = np.full(blocks.shape[:-1] + (C * ppb,), -1, dtype=np.int32)
    for b in range(w.batch):
        L_ = int(x.seqlens[b])
        for idx in np.ndindex(*blocks.shape[1:-1]):
            row = blocks[(b,) + idx]
            n_ = int((row >= 0).sum())
            pages[(b,) + idx][:n_ * ppb] = expected_pages(row[:n_], x.page_table[b], ppb,
                                                          w.block, L_)
    mask = bk.OrderedMask(blocks=torch.from_numpy(blocks).to(DEV),
                          pages=torch.from_numpy(pages).to(DEV),
                          counts=torch.from_numpy(counts).to(DEV), hrm_counts=None, capacity=C)
    if shared:
        res = bk.osk_prefill_shared_kv(prob, q, k, v, mask, tau)
        # the oracle walks each query head's copy of its KV head's row
        grp_ = w.num_q_heads // w.num_kv_heads
        blocks, counts = np.repeat(blocks, grp_, axis=1), np.repeat(counts, grp_, axis=1)
    elif delta is None:
        res = bk.osk_prefill(prob, q, k, v, mask, tau)
    else:
        res = bk.osk_prefill_delta(prob, q, k, v, mask, delta)
    torch.cuda.synchronize()
    out, lse, rec, stats = _np(res.out), _np(res.lse), _np(res.skip_record), _np(res.row_stats)
    st, ls = ErrStats(), ErrStats()
    near_total = 0
    n_skipped = 0
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        s0, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        if L == 0:
            continue
        kk = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        vv = materialise(x.v_pool, x.page_table[b], L, w.page_size)
        nqb = (L + w.q_block - 1) // w.q_block
        if delta is None:
            tau_b, on = tau, tau >= 0
        else:
            on = delta > 0
            tau_b = oosk.tau_from_delta(L, delta) if on else -1.0
        for h in range(w.num_q_heads):
            g = h // grp
            for i in range(nqb):
                if tiles is not None and (b, h, i) not in tiles:
                    continue
                rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
                cnt = int(counts[b, h, i])
                bl = blocks[b, h, i, :cnt]
                qr = x.q[s0 + rows, h].astype(np.float64)
                r = oosk.osk_tile_closed_form(qr, rows, kk[:, g], vv[:, g], bl, tau_b,
                                              w.softmax_scale, w.block, skip_on=on)
                near_total += check_osk_tile(out[s0 + rows, h], lse[h, s0 + rows],
                                             rec[b, h, i], r, qr, rows, kk[:, g], vv[:, g], bl,
                                             w.softmax_scale, w.block, st, ls)
                n_skipped += int(rec[b, h, i, :cnt].sum())
                assert stats[b, h, i, 0] == cnt
                assert stats[b, h, i, 1] == int(rec[b, h, i, :cnt].sum())
    report(label, skipped=n_skipped, near_threshold=near_total)
    st.assert_ok(label=f"{label} out")
    ls.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"{label} lse")
    return n_skipped


@pytest.mark.parametrize("case", [("tiny", {}), ("tiny", dict(RAGGED))])
def test_osk_full_budget_skip_off_equals_dense(case):
    name, kw = case
    w, x = _inputs(name, **kw)
    print(f"[case] osk full budget {name} {kw}", flush=True)
    blocks, counts = oosk.dense_order_mask(x.cu_seqlens, w.num_q_heads, w.q_block, w.block)
    _run_osk_vs_oracle(w, x, blocks, counts, -1.0, f"osk-full {name}")


@pytest.mark.parametrize("seqlens", [RAGGED["seqlens"], (9000, 20000, 130)])
def test_osk_every_block_ascending_equals_dense_bitwise(seqlens):
    # The ordered walk over every causal block in ascending order with the skip
    # off visits what the dense walk visits, in the same order, with the same
    # arithmetic: the outputs and LSE agree bit for bit (the dense kernel pairs
    # two query heads per workgroup in opposite phases; the ordered kernel runs
    # one head per workgroup).  The longer sequences refill the slot rings.
    w, x = _inputs("tiny", **dict(RAGGED, seqlens=seqlens, num_q_heads=4, num_kv_heads=2))
    print(f"[case] osk ascending every block vs dense, seqlens={seqlens}", flush=True)
    prob, q, k, v = upload(x, DEV)
    blocks, counts = oosk.dense_order_mask(x.cu_seqlens, w.num_q_heads, w.q_block, w.block)
    C = blocks.shape[-1]
    pages = np.full(blocks.shape, -1, dtype=np.int32)
    for b in range(w.batch):
        for idx in np.ndindex(*blocks.shape[1:-1]):
            row = blocks[(b,) + idx]
            n_ = int((row >= 0).sum())
            pages[(b,) + idx][:n_] = x.page_table[b][row[:n_]]
    mask = bk.OrderedMask(blocks=torch.from_numpy(blocks).to(DEV),
                          pages=torch.from_numpy(pages).to(DEV),
                          counts=torch.from_numpy(counts).to(DEV), hrm_counts=None, capacity=C)
    o = bk.osk_prefill(prob, q, k, v, mask, -1.0)
    d = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(d.out.float()).any())
    assert torch.equal(o.out, d.out)
    assert torch.equal(o.lse, d.lse)
    report(f"osk ascending = dense {seqlens}", tiles=int((counts > 0).sum()),
           max_blocks=int(counts.max()))


@pytest.mark.parametrize("tau", [-1.0, 0.0, 4.0, 8.0])
def test_osk_oracle_mask_with_skip(tau):
    w, x = _inputs("tiny_skip")
    print(f"[case] osk tiny_skip tau={tau}", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, w.budget, w.softmax_scale)
    n = _run_osk_vs_oracle(w, x, m.blocks, m.counts, tau, f"osk tiny_skip tau={tau}")
    if 0 <= tau <= 8:
        assert n > 0


def test_osk_any_order_same_output():
    # reversed and shuffled visiting orders of the same set, skip off
    w, x = _inputs("tiny", **RAGGED)
    print("[case] osk any-order", flush=True)
    blocks, counts = oosk.dense_order_mask(x.cu_seqlens, w.num_q_heads, w.q_block, w.block)
    rng = np.random.default_rng(0)
    sh = blocks.copy()
    for idx in np.ndindex(*counts.shape):
        c = counts[idx]
        sh[idx][:c] = rng.permutation(sh[idx][:c])
    _run_osk_vs_oracle(w, x, sh, counts, -1.0, "osk shuffled order")


def test_osk_ragged_small_budget_with_kap_order():
    w, x = _inputs("tiny", **dict(RAGGED, q_dir_gain=6.0))
    print("[case] osk ragged budget 0.2", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, 0.2, w.softmax_scale)
    _run_osk_vs_oracle(w, x, m.blocks, m.counts, 2.0, "osk ragged b=0.2 tau=2")


def _kap_compare(w, x, budget, label, tiles=None, debug=True):
    prob, q, k, v = upload(x, DEV)
    gm = bk.proxy_ordered_mask(prob, q, k, budget, debug=debug)
    torch.cuda.synchronize()
    gb, gp, gc, gh = _np(gm.blocks), _np(gm.pages), _np(gm.counts), _np(gm.hrm_counts)
    dw = _np(gm.debug_w) if debug else None
    dh = _np(gm.debug_hrm) if debug else None
    beta = okap.budget_ppm(budget)
    assert gm.capacity == okap.mask_capacity(int(max(w.seqlens)), w.block, beta)
    exact = ties = own = 0
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        s0, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        nqb = (L + w.q_block - 1) // w.q_block
        assert np.all(gc[b, :, nqb:] == 0)
        assert np.all(gb[b, :, nqb:] == -1)
        if L == 0:
            continue
        kk = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        for h in range(w.num_q_heads):
            want = None if tiles is None else [i for (bb, hh, i) in tiles if bb == b and hh == h]
            if want is not None and not want:
                continue
            res = okap.head_tiles(x.q[s0:s0 + L, h].astype(np.float64), kk[:, h // grp],
                                  w.softmax_scale, w.q_block, w.block, beta, tiles=want)
            for i, tile in res.items():
                if debug:
                    # bit-exact: the selection rule on the kernel's own w and flags
                    want = selection_on_own_scores(dw[b, h, i], dh[b, h, i], tile.n, beta)
                    c = int(gc[b, h, i])
                    assert c == len(want) and np.array_equal(gb[b, h, i, :c], want), (b, h, i)
                    own += 1
                kind = check_kap_row(gb[b, h, i], gp[b, h, i], gc[b, h, i], gh[b, h, i], tile,
                                     x.page_table[b], ppb=w.block // w.page_size,
                                     kv_block=w.block, L=L)
                exact += kind == "exact"
                ties += kind == "tie"
    report(label, own_score_exact=own, exact=exact, near_tie=ties)
    return gm, exact, ties


@pytest.mark.parametrize("case", [("tiny", {}, 0.5), ("tiny_skip", {}, 0.5),
                                  ("tiny", dict(RAGGED), 0.3), ("tiny", dict(RAGGED), 1.0),
                                  ("tiny", dict(RAGGED, q_block=64), 0.05),
                                  ("tiny", dict(RAGGED, head_dim=64), 0.3)])
def test_kap_matches_oracle(case):
    name, kw, budget = case
    w, x = _inputs(name, **kw)
    print(f"[case] kap {name} {kw} budget={budget}", flush=True)
    _, exact, ties = _kap_compare(w, x, budget, f"kap {name} b={budget}")
    assert exact > 0 and ties <= max(1, exact // 100)


def test_deterministic_and_poison_safe():
    w, x = _inputs("tiny", **RAGGED)
    print("[case] determinism", flush=True)
    prob, q, k, v = upload(x, DEV)
    outs = []
    for _ in range(2):
        m = bk.proxy_ordered_mask(prob, q, k, 0.3)
        r = bk.osk_prefill(prob, q, k, v, m, 4.0)
        d = bk.dense_prefill(prob, q, k, v)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (m.blocks, m.pages, m.counts, r.out, r.lse,
                                          r.skip_record, d.out, d.lse)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    # the pool's spare pages and the tails of last pages hold NaN
    assert np.isnan(x.k_pool).any()
    for t in (outs[0][3], outs[0][6]):
        assert torch.isfinite(t.float()).all()


# ---------------------------------------------------------------------------
# Length-adaptive threshold Delta / N (cosa_osk_prefill_delta)

SKIP_RAGGED = dict(seqlens=(700, 1500, 90), shuffled_pages=True, spare_pages=5,
                   precision="bf16")


@pytest.mark.parametrize("delta", [-1.0, 50.0, 200.0, 2000.0])
def test_osk_delta_per_sequence_threshold(delta):
    # tau_b = ln(L_b / delta): 2.64 / 3.40 / 0.59 nats at delta 50 and negative
    # (skip still on) for the shorter sequences at delta 2000
    w, x = _inputs("tiny_skip", **SKIP_RAGGED)
    print(f"[case] osk delta={delta} seqlens={w.seqlens}", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, w.budget, w.softmax_scale)
    n = _run_osk_vs_oracle(w, x, m.blocks, m.counts, 0.0, f"osk delta={delta}", delta=delta)
    if delta > 0:
        assert n > 0
    else:
        assert n == 0


# ---------------------------------------------------------------------------
# Stage-1 Top-p (cosa_proxy_ordered_mask_top_p)

TOP_P_TOL = 1e-5   # fp32 importance scores against fp64: mass near-ties


def _allowed_counts(tile, top_p, beta_ppm):
    kb = okap.budget_count(tile.n, beta_ppm)
    if top_p >= 1.0:
        return {kb}
    cum = np.concatenate([[0.0], np.cumsum(tile.w[tile.order])])
    ok = {tile.k}
    for kp in range(1, tile.n + 1):
        if cum[kp - 1] < top_p + TOP_P_TOL and cum[kp] >= top_p - TOP_P_TOL:
            ok.add(min(kb, kp))
    return ok


@pytest.mark.parametrize("case", [("tiny", {}, 0.5, 1.0), ("tiny", {}, 0.95, 1.0),
                                  ("tiny_skip", {}, 0.8, 1.0), ("tiny", dict(RAGGED), 0.9, 0.3),
                                  ("tiny", dict(RAGGED, q_block=64), 0.95, 1.0),
                                  ("tiny", dict(RAGGED), 1.0, 0.5)])
def test_kap_top_p_matches_oracle(case):
    name, kw, top_p, cap = case
    w, x = _inputs(name, **kw)
    print(f"[case] kap top_p={top_p} cap={cap} {name} {kw}", flush=True)
    prob, q, k, v = upload(x, DEV)
    gm = bk.proxy_ordered_mask_top_p(prob, q, k, top_p, cap, debug=True)
    torch.cuda.synchronize()
    gb, gp, gc, gh = _np(gm.blocks), _np(gm.pages), _np(gm.counts), _np(gm.hrm_counts)
    dw, dh = _np(gm.debug_w), _np(gm.debug_hrm)
    beta = okap.budget_ppm(cap)
    exact = ties = shorter = 0
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        s0, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        nqb = (L + w.q_block - 1) // w.q_block
        assert np.all(gc[b, :, nqb:] == 0)
        if L == 0:
            continue
        kk = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        for h in range(w.num_q_heads):
            res = okap.head_tiles(x.q[s0:s0 + L, h].astype(np.float64), kk[:, h // grp],
                                  w.softmax_scale, w.q_block, w.block, beta, top_p=top_p)
            for i, tile in res.items():
                c = int(gc[b, h, i])
                # 1) bit-exact: the documented rule on the kernel's own w and flags
                want = selection_on_own_scores(dw[b, h, i], dh[b, h, i], tile.n, beta, top_p)
                assert c == len(want) and np.array_equal(gb[b, h, i, :c], want), (b, h, i)
                # 2) against the fp64 oracle: the count up to mass near-ties,
                #    then the kept blocks as for the budget mask
                assert c in _allowed_counts(tile, top_p, beta), (b, h, i, c, tile.k)
                shorter += c < tile.n
                kind = check_kap_row(gb[b, h, i], gp[b, h, i], c, gh[b, h, i],
                                     dataclasses.replace(tile, k=c), x.page_table[b])
                exact += kind == "exact" and c == tile.k
                ties += kind == "tie" or c != tile.k
    report(f"kap top_p={top_p} cap={cap}", own_score_exact=exact + ties, exact=exact,
           near_tie=ties, truncated=shorter)
    assert exact > 0 and ties <= max(1, exact // 100)
    if top_p < 1.0:
        assert shorter > 0


# ---------------------------------------------------------------------------
# Remapping ablation and logical mask skipping


def test_osk_ascending_order_of_kap_set_with_skip():
    # the KAP kept sets visited in ascending block order (no remapping), skip on
    w, x = _inputs("tiny_skip")
    print("[case] osk ascending kap set tau=4", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, w.budget, w.softmax_scale)
    asc = m.blocks.copy()
    for idx in np.ndindex(*m.counts.shape):
        c = m.counts[idx]
        asc[idx][:c] = np.sort(asc[idx][:c])
    _run_osk_vs_oracle(w, x, asc, m.counts, 4.0, "osk ascending tau=4")


@pytest.mark.parametrize("case", [("tiny", dict(RAGGED), 0.3), ("tiny_skip", {}, 0.2),
                                  ("tiny", dict(RAGGED, q_block=64, head_dim=64), 0.5)])
def test_block_mask_logical_skip_matches_oracle(case):
    from block_sparse_long_kap_amd.masks import block_bitmask
    name, kw, budget = case
    w, x = _inputs(name, **kw)
    print(f"[case] logical skip {name} {kw} budget={budget}", flush=True)
    prob, q, k, v = upload(x, DEV)
    gm = bk.proxy_ordered_mask(prob, q, k, budget)
    bits = block_bitmask(prob, gm)
    res = bk.block_mask_prefill(prob, q, k, v, bits)
    osk = bk.osk_prefill(prob, q, k, v, gm, -1.0)
    torch.cuda.synchronize()
    out, lse = _np(res.out), _np(res.lse)
    gb, gc = _np(gm.blocks), _np(gm.counts)
    st, ls = ErrStats(), ErrStats()
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        s0, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        if L == 0:
            continue
        kk = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        vv = materialise(x.v_pool, x.page_table[b], L, w.page_size)
        for h in range(w.num_q_heads):
            for i in range((L + w.q_block - 1) // w.q_block):
                rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
                key_ok = np.zeros(L, dtype=bool)
                for j in gb[b, h, i, :gc[b, h, i]]:
                    key_ok[j * w.block:min((j + 1) * w.block, L)] = True
                o, l_ = odense.attention_rows(x.q[s0 + rows, h].astype(np.float64), rows,
                                              kk[:, h // grp], vv[:, h // grp], w.softmax_scale,
                                              key_ok=key_ok)
                st.add(out[s0 + rows, h], o)
                fin = np.isfinite(l_)
                assert np.array_equal(np.isfinite(lse[h, s0 + rows]), fin)
                ls.add(lse[h, s0 + rows][fin], l_[fin])
    st.assert_ok(label=f"logical skip {name} out")
    ls.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"logical skip {name} lse")
    # the same set through the OSK (skip off) agrees with it to rounding order
    d = np.abs(_np(osk.out).astype(np.float64) - out)
    assert d.max() <= 2e-2


# ---------------------------------------------------------------------------
# KV-group-shared masks (cosa_proxy_ordered_mask_shared_kv, cosa_osk_prefill_shared_kv)


@pytest.mark.parametrize("case", [("tiny", dict(RAGGED), 0.3, 1.0),
                                  ("tiny", dict(RAGGED, q_block=64), 0.2, 1.0),
                                  ("tiny", dict(RAGGED, num_q_heads=4), 0.5, 1.0),
                                  ("tiny", dict(RAGGED), 1.0, 0.9),
                                  ("tiny_skip", {}, 0.5, 1.0),
                                  # eight query heads per mask (four proxy rows each)
                                  ("tiny", dict(RAGGED, num_q_heads=16, q_block=64), 0.3, 1.0),
                                  ("tiny", dict(RAGGED, head_dim=64), 0.3, 1.0)])
def test_kap_shared_kv_matches_oracle(case):
    name, kw, budget, top_p = case
    w, x = _inputs(name, **kw)
    print(f"[case] kap shared {name} {kw} budget={budget} top_p={top_p}", flush=True)
    prob, q, k, v = upload(x, DEV)
    gm = bk.proxy_ordered_mask_shared_kv(prob, q, k, budget, top_p, debug=True)
    torch.cuda.synchronize()
    gb, gp, gc, gh = _np(gm.blocks), _np(gm.pages), _np(gm.counts), _np(gm.hrm_counts)
    dw, dh = _np(gm.debug_w), _np(gm.debug_hrm)
    beta = okap.budget_ppm(budget)
    grp = w.num_q_heads // w.num_kv_heads
    assert gb.shape[1] == w.num_kv_heads
    exact = ties = 0
    tp = None if top_p >= 1.0 else top_p
    for b in range(w.batch):
        s0, L = int(x.cu_seqlens[b]), int(x.seqlens[b])
        nqb = (L + w.q_block - 1) // w.q_block
        assert np.all(gc[b, :, nqb:] == 0)
        if L == 0:
            continue
        kk = materialise(x.k_pool, x.page_table[b], L, w.page_size)
        for g in range(w.num_kv_heads):
            qs = [x.q[s0:s0 + L, h].astype(np.float64) for h in range(g * grp, (g + 1) * grp)]
            res = okap.group_tiles(qs, kk[:, g], w.softmax_scale, w.q_block, w.block, beta,
                                   top_p=tp)
            for i, tile in res.items():
                c = int(gc[b, g, i])
                want = selection_on_own_scores(dw[b, g, i], dh[b, g, i], tile.n, beta,
                                              1.0 if tp is None else tp)
                assert c == len(want) and np.array_equal(gb[b, g, i, :c], want), (b, g, i)
                if tp is not None:
                    assert c in _allowed_counts(tile, tp, beta), (b, g, i, c, tile.k)
                kind = check_kap_row(gb[b, g, i], gp[b, g, i], c, gh[b, g, i],
                                     dataclasses.replace(tile, k=c), x.page_table[b])
                exact += kind == "exact" and c == tile.k
                ties += kind == "tie" or c != tile.k
    report(f"kap shared {name}", exact=exact, near_tie=ties)
    assert exact > 0 and ties <= max(1, exact // 100)


@pytest.mark.parametrize("tau", [-1.0, 4.0])
def test_osk_shared_kv_masks(tau):
    w, x = _inputs("tiny", **dict(RAGGED, q_dir_gain=6.0))
    print(f"[case] osk shared masks tau={tau}", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, 0.3, w.softmax_scale, shared_kv=True)
    _run_osk_vs_oracle(w, x, m.blocks, m.counts, tau, f"osk shared tau={tau}", shared=True)


# ---------------------------------------------------------------------------
# Logical key blocks of 128 keys resolved through two 64-token pages


KV128 = dict(RAGGED, kv_block=128, seqlens=(1, 63, 64, 65, 127, 128, 129, 200, 383))
# every (head_dim, q_block) instance of the two-page kernel (wavefront pairs
# of 4 or 2 row groups)
KV128_SHAPES = [(128, 128), (128, 64), (64, 128), (64, 64)]


@pytest.mark.parametrize("head_dim,q_block", KV128_SHAPES)
def test_dense_kv_block_128_matches_oracle(head_dim, q_block):
    w, x = _inputs("tiny", **dict(KV128, head_dim=head_dim, q_block=q_block))
    print(f"[case] dense kv_block=128 D={head_dim} q_block={q_block}", flush=True)
    prob, q, k, v = upload(x, DEV)
    res = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    ref, ref_lse = _dense_oracle(x, w)
    st, ls = ErrStats(), ErrStats()
    st.add(_np(res.out), ref)
    ls.add(_np(res.lse), ref_lse)
    st.assert_ok(label="dense kv_block=128 out")
    ls.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="dense kv_block=128 lse")


@pytest.mark.parametrize("head_dim,q_block", KV128_SHAPES)
def test_osk_kv_block_128_full_budget_and_shuffled(head_dim, q_block):
    w, x = _inputs("tiny", **dict(KV128, head_dim=head_dim, q_block=q_block))
    print(f"[case] osk kv_block=128 D={head_dim} q_block={q_block} full budget, shuffled",
          flush=True)
    blocks, counts = oosk.dense_order_mask(x.cu_seqlens, w.num_q_heads, w.q_block, w.block)
    _run_osk_vs_oracle(w, x, blocks, counts, -1.0, "osk kv128 full")
    rng = np.random.default_rng(1)
    sh = blocks.copy()
    for idx in np.ndindex(*counts.shape):
        c = counts[idx]
        sh[idx][:c] = rng.permutation(sh[idx][:c])
    _run_osk_vs_oracle(w, x, sh, counts, -1.0, "osk kv128 shuffled")


@pytest.mark.parametrize("budget", [0.3, 1.0])
def test_kap_kv_block_128_matches_oracle(budget):
    w, x = _inputs("tiny", **KV128)
    print(f"[case] kap kv_block=128 budget={budget}", flush=True)
    _, exact, ties = _kap_compare(w, x, budget, f"kap kv128 b={budget}")
    assert exact > 0 and ties <= max(1, exact // 100)


@pytest.mark.parametrize("tau", [0.0, 4.0, 8.0])
def test_osk_kv_block_128_with_skip(tau):
    w, x = _inputs("tiny_skip", kv_block=128, seqlens=(700, 1500, 90), shuffled_pages=True,
                   spare_pages=5, precision="bf16")
    print(f"[case] osk kv_block=128 tiny_skip tau={tau}", flush=True)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, w.budget, w.softmax_scale)
    n = _run_osk_vs_oracle(w, x, m.blocks, m.counts, tau, f"osk kv128 tau={tau}")
    assert n > 0


# ---------------------------------------------------------------------------
# Degenerate inputs: empty sequences in the batch, a budget that keeps one
# block per tile, tau = 0, and every entry point on the same batch


EMPTY = dict(seqlens=(0, 100, 0, 257, 1), num_q_heads=4, num_kv_heads=2, head_dim=64,
             q_block=64, precision="bf16", shuffled_pages=True, spare_pages=3)


def test_empty_sequences_and_single_block_budget():
    w, x = _inputs("tiny", **EMPTY)
    print("[case] empty sequences, budget keeping one block", flush=True)
    prob, q, k, v = upload(x, DEV)
    _, exact, ties = _kap_compare(w, x, 1e-6, "kap one block")
    assert exact > 0 and ties == 0
    gm = bk.proxy_ordered_mask(prob, q, k, 1e-6)
    torch.cuda.synchronize()
    gc = _np(gm.counts)
    for b, L in enumerate(x.seqlens):
        nqb = (int(L) + w.q_block - 1) // w.q_block
        assert np.all(gc[b, :, :nqb] == 1) and np.all(gc[b, :, nqb:] == 0)
    m = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                w.q_block, w.block, 1e-6, w.softmax_scale)
    _run_osk_vs_oracle(w, x, m.blocks, m.counts, 0.0, "osk one block tau=0")
    # dense and shared masks on the same batch
    res = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    ref, ref_lse = _dense_oracle(x, w)
    st = ErrStats()
    st.add(_np(res.out), ref)
    st.assert_ok(label="dense with empty sequences")
    ms = okap.proxy_ordered_mask(x.q, x.k_pool, x.page_table, x.cu_seqlens, w.num_kv_heads,
                                 w.q_block, w.block, 0.5, w.softmax_scale, shared_kv=True)
    _run_osk_vs_oracle(w, x, ms.blocks, ms.counts, 4.0, "osk shared, empty sequences",
                       shared=True)


@pytest.mark.parametrize("case", [
    ("tiny_skip", {}, 0.5, 2.0),
    # 6 sequences x 2 KV heads = 12 groups, one chunk at this size
    ("tiny", dict(RAGGED, q_dir_gain=6.0), 0.2, 2.0),
    # 4 sequences x 8 KV heads = 32 groups of 2048 workgroups (64K tokens): eight
    # chunks of 4 groups, two of them on the empty sequence; the skip fires
    ("remap32k", dict(seqlens=(65536, 0, 3000, 40000)), 0.3, 6.0),
    ("tiny", dict(RAGGED, seqlens=(1500, 0, 700, 2047), num_kv_heads=4), 0.3, -1.0),
    # 128-key logical blocks over two pages
    ("tiny_skip", dict(kv_block=128), 0.5, 2.0),
])
@pytest.mark.parametrize("aux", [False, True])
def test_fused_proxy_and_kernel_equal_separate_calls(case, aux):
    """cosa_sparse_prefill gives, bit for bit, what cosa_proxy_ordered_mask followed by
    cosa_osk_prefill give, on one stream and with the kernel on a second stream."""
    name, kw, budget, tau = case
    w, x = _inputs(name, **kw)
    print(f"[case] fused {name} {kw} budget={budget} tau={tau} aux={aux}", flush=True)
    prob, q, k, v = upload(x, DEV)
    m1 = bk.proxy_ordered_mask(prob, q, k, budget)
    r1 = bk.osk_prefill(prob, q, k, v, m1, tau, record=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV) if aux else None
    # poison the outputs so that anything the fused call fails to write shows
    m2 = bk.proxy_ordered_mask(prob, q, k, budget)
    r2 = bk.osk_prefill(prob, q, k, v, m2, tau, record=True)
    for t in (m2.blocks, m2.pages, m2.counts, m2.hrm_counts, r2.row_stats):
        t.fill_(-7)
    r2.out.fill_(float("nan"))
    r2.lse.fill_(float("nan"))
    r2.skip_record.fill_(9)
    m2, r2 = bk.sparse_prefill(prob, q, k, v, budget, tau, aux_stream=side, mask=m2, out=r2)
    torch.cuda.synchronize()
    for a, b_ in ((m1.blocks, m2.blocks), (m1.pages, m2.pages), (m1.counts, m2.counts),
                  (m1.hrm_counts, m2.hrm_counts), (r1.row_stats, r2.row_stats)):
        assert torch.equal(a, b_)
    assert torch.equal(r1.out.view(torch.int16), r2.out.view(torch.int16))
    assert torch.equal(r1.lse.view(torch.int32), r2.lse.view(torch.int32))
    # the skip record: equal on every slot below the count (the rest is untouched)
    cnt = m1.counts.reshape(-1).cpu().numpy()
    s1 = r1.skip_record.reshape(cnt.size, -1).cpu().numpy()
    s2 = r2.skip_record.reshape(cnt.size, -1).cpu().numpy()
    for row, c in enumerate(cnt):
        assert np.array_equal(s1[row, :c], s2[row, :c])
