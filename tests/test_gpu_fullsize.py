"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The whole layer runs on the GPU (proxy ordered mask -> ordered-skipping
prefill, and the dense kernel); the CPU oracle then recomputes a seeded
sample of (head, tile) pairs one by one - their mask rows, their OSK outputs,
skip decisions and their dense outputs - and the GPU values at those pairs are
compared with it.  Layer-wide properties (counts, capacity, page remap,
finiteness) are checked everywhere.
"""
import numpy as np
import pytest

import block_sparse_long_kap_amd as bk
import cosa_inputs as ci
from oracle import dense as odense
from oracle import kap as okap
from oracle import osk as oosk
from oracle.paging import materialise

from .parity import (MAX_ABS, MEAN_ABS, ErrStats, check_kap_row, check_osk_tile, report,
                     selection_on_own_scores, upload)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _sample(w, x, n, seed):
    rng = np.random.default_rng(seed)
    picks = []
    lens = np.diff(x.cu_seqlens)
    for _ in range(n):
        b = int(rng.integers(w.batch))
        nqb = (int(lens[b]) + w.q_block - 1) // w.q_block
        picks.append((b, int(rng.integers(w.num_q_heads)), int(rng.integers(nqb))))
    # always include the longest tile and the first tile of the longest sequence
    bl = int(np.argmax(lens))
    nq = (int(lens[bl]) + w.q_block - 1) // w.q_block
    picks += [(bl, 0, nq - 1), (bl, w.num_q_heads - 1, 0)]
    return sorted(set(picks))


@pytest.mark.parametrize("name,n_samples", [("llama32k", 24), ("llama128k", 10),
                                            ("qwen128k", 10), ("stress", 12)])
def test_full_layer_sampled_parity(name, n_samples):
    w = ci.get(name)
    print(f"[case] full-size {name}: generating inputs", flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    print(f"[case] full-size {name}: GPU layer", flush=True)
    # the proxy instance bench.py times (the score export is a runtime option
    # of the same kernel)
    m = bk.proxy_ordered_mask(prob, q, k, w.budget, debug=True)
    r = bk.osk_prefill(prob, q, k, v, m, w.tau)
    torch.cuda.synchronize()
    # the fused call at full size, the kernel on a second stream: same bits
    print(f"[case] full-size {name}: fused call", flush=True)
    fm, fr = bk.sparse_prefill(prob, q, k, v, w.budget, w.tau,
                               aux_stream=torch.cuda.Stream(DEV))
    torch.cuda.synchronize()
    assert torch.equal(fm.blocks, m.blocks) and torch.equal(fm.counts, m.counts)
    assert torch.equal(fm.pages, m.pages) and torch.equal(fm.hrm_counts, m.hrm_counts)
    assert torch.equal(fr.out.view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(fr.lse.view(torch.int32), r.lse.view(torch.int32))
    assert torch.equal(fr.row_stats, r.row_stats)
    del fm, fr
    gb, gp, gc, gh = _np(m.blocks), _np(m.pages), _np(m.counts), _np(m.hrm_counts)
    dw, dh = _np(m.debug_w), _np(m.debug_hrm)
    out, lse, rec, stats = _np(r.out), _np(r.lse), _np(r.skip_record), _np(r.row_stats)
    del r
    d = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    dout, dlse = _np(d.out), _np(d.lse)
    del d, q, k, v
    beta = okap.budget_ppm(w.budget)
    lens = np.diff(x.cu_seqlens)
    # layer-wide checks
    assert m.capacity == okap.mask_capacity(int(lens.max()), w.page_size, beta)
    for b in range(w.batch):
        nqb = (int(lens[b]) + w.q_block - 1) // w.q_block
        n_i = (np.minimum((np.arange(nqb) + 1) * w.q_block, lens[b]) - 1) // w.page_size + 1
        want = np.array([okap.budget_count(int(n), beta) for n in n_i])
        assert np.all(gc[b, :, :nqb] == want[None, :])
        assert np.all(gc[b, :, nqb:] == 0)
        sel = gb[b] >= 0
        assert np.array_equal(gp[b][sel], x.page_table[b][gb[b][sel]])
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(dout))
    assert np.array_equal(stats[..., 0], gc)
    # bit-exact: the selection rule on the kernel's own scores, on a seeded
    # sample of mask rows (plus every row the oracle checks below)
    picks = _sample(w, x, n_samples, seed=w.seed)
    rng = np.random.default_rng(w.seed + 100)
    own_rows = set(picks)
    for _ in range(512):
        b = int(rng.integers(w.batch))
        own_rows.add((b, int(rng.integers(w.num_q_heads)),
                      int(rng.integers((int(lens[b]) + w.q_block - 1) // w.q_block))))
    for (b, h, i) in sorted(own_rows):
        n = (min((i + 1) * w.q_block, int(lens[b])) - 1) // w.page_size + 1
        want = selection_on_own_scores(dw[b, h, i], dh[b, h, i], n, beta)
        c = int(gc[b, h, i])
        assert c == len(want) and np.array_equal(gb[b, h, i, :c], want), (b, h, i)
    del dw, dh
    # sampled oracle checks
    grp = w.num_q_heads // w.num_kv_heads
    kap_exact = kap_tie = 0
    so, sl, do, dl = ErrStats(), ErrStats(), ErrStats(), ErrStats()
    near = 0
    cache = {}
    print(f"[case] full-size {name}: oracle on {len(picks)} tiles", flush=True)
    for (b, h, i) in picks:
        s0, L = int(x.cu_seqlens[b]), int(lens[b])
        if b not in cache:
            cache = {b: (materialise(x.k_pool, x.page_table[b], L, w.page_size),
                         materialise(x.v_pool, x.page_table[b], L, w.page_size))}
        kk, vv = cache[b]
        g = h // grp
        tile = okap.head_tiles(x.q[s0:s0 + L, h].astype(np.float64), kk[:, g], w.softmax_scale,
                               w.q_block, w.page_size, beta, tiles=[i])[i]
        kind = check_kap_row(gb[b, h, i], gp[b, h, i], gc[b, h, i], gh[b, h, i], tile,
                             x.page_table[b])
        kap_exact += kind == "exact"
        kap_tie += kind == "tie"
        rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
        qr = x.q[s0 + rows, h].astype(np.float64)
        # OSK on the GPU's own mask row (equal to the oracle's, or a near-tie variant of it)
        bl = gb[b, h, i, :gc[b, h, i]]
        res = oosk.osk_tile_closed_form(qr, rows, kk[:, g], vv[:, g], bl, w.tau,
                                        w.softmax_scale, w.page_size)
        near += check_osk_tile(out[s0 + rows, h], lse[h, s0 + rows], rec[b, h, i], res, qr,
                               rows, kk[:, g], vv[:, g], bl, w.softmax_scale, w.page_size, so,
                               sl)
        o, ls = odense.attention_rows(qr, rows, kk[:, g], vv[:, g], w.softmax_scale)
        do.add(dout[s0 + rows, h], o)
        dl.add(dlse[h, s0 + rows], ls)
    report(f"full-size {name}", own_score_exact=len(own_rows), kap_exact=kap_exact,
           kap_near_tie=kap_tie, osk_near_threshold=near,
           layer_skipped=int(stats[..., 1].sum()), layer_visited=int(stats[..., 0].sum()))
    so.assert_ok(label=f"{name} osk out")
    sl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"{name} osk lse")
    do.assert_ok(label=f"{name} dense out")
    dl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"{name} dense lse")
    assert kap_exact >= len(picks) // 2


def test_full_layer_shared_kv_sampled_parity():
    """llama128k with one mask per KV head (cosa_proxy_ordered_mask_shared_kv +
    cosa_osk_prefill_shared_kv, as timed by bench.py --shared-kv), sampled."""
    w = ci.get("llama128k")
    print("[case] full-size shared-kv llama128k: generating inputs", flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    print("[case] full-size shared-kv llama128k: GPU layer", flush=True)
    m = bk.proxy_ordered_mask_shared_kv(prob, q, k, w.budget)
    r = bk.osk_prefill_shared_kv(prob, q, k, v, m, w.tau)
    torch.cuda.synchronize()
    gb, gp, gc, gh = _np(m.blocks), _np(m.pages), _np(m.counts), _np(m.hrm_counts)
    out, lse, rec = _np(r.out), _np(r.lse), _np(r.skip_record)
    del r, q, k, v
    assert gb.shape[1] == w.num_kv_heads and np.all(np.isfinite(out))
    beta = okap.budget_ppm(w.budget)
    grp = w.num_q_heads // w.num_kv_heads
    L = int(x.seqlens[0])
    kk = materialise(x.k_pool, x.page_table[0], L, w.page_size)
    vv = materialise(x.v_pool, x.page_table[0], L, w.page_size)
    rng = np.random.default_rng(11)
    nqb = (L + w.q_block - 1) // w.q_block
    picks = sorted({(int(rng.integers(w.num_kv_heads)), int(rng.integers(nqb))) for _ in range(6)}
                   | {(0, nqb - 1)})
    so, sl = ErrStats(), ErrStats()
    exact = near = 0
    for g, i in picks:
        qs = [x.q[:L, h].astype(np.float64) for h in range(g * grp, (g + 1) * grp)]
        tile = okap.group_tiles(qs, kk[:, g], w.softmax_scale, w.q_block, w.page_size, beta,
                                tiles=[i])[i]
        exact += check_kap_row(gb[0, g, i], gp[0, g, i], gc[0, g, i], gh[0, g, i], tile,
                               x.page_table[0]) == "exact"
        bl = gb[0, g, i, :gc[0, g, i]]
        rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
        for h in (g * grp, g * grp + grp - 1):
            qr = x.q[rows, h].astype(np.float64)
            res = oosk.osk_tile_closed_form(qr, rows, kk[:, g], vv[:, g], bl, w.tau,
                                            w.softmax_scale, w.page_size)
            near += check_osk_tile(out[rows, h], lse[h, rows], rec[0, h, i], res, qr, rows,
                                   kk[:, g], vv[:, g], bl, w.softmax_scale, w.page_size, so, sl)
    report("full-size shared-kv llama128k", kap_exact=exact, kap_rows=len(picks),
           osk_near_threshold=near)
    so.assert_ok(label="shared-kv osk out")
    sl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="shared-kv osk lse")
    assert exact >= len(picks) // 2


# ---------------------------------------------------------------------------
# The in-kernel skip on long tiles.  The kernel reads each tile's slot
# lookups from a ring of two 64-slot chunks in LDS and refills a chunk from
# memory every 64 slots; tiles with more than 128 visited blocks take that
# refill, and a computed block right after a skipped one fetches its V page
# on demand.  These cases make the skip fire on such tiles at full size.


def _refill_after_skip(gc, rec):
    """Mask rows (b, h, i) with a slot 64c - 1 (c >= 1) that is computed right
    after a skipped slot while a later chunk of the ring is still refilled
    (64 (c + 1) < count)."""
    hit = np.zeros(gc.shape, dtype=bool)
    C = rec.shape[-1]
    for c in range(1, C // 64 + 1):
        t = 64 * c - 1
        if t >= C:
            break
        hit |= (gc > 64 * (c + 1)) & (rec[..., t - 1] == 1) & (rec[..., t] == 0)
    return hit


def _long_tile_picks(w, gc, rec, stats, seed):
    rng = np.random.default_rng(seed)
    B, H, _ = gc.shape
    picks = set()
    # the longest tile of four heads of every sequence
    for b in range(B):
        i_long = int(np.argmax(gc[b, 0]))
        for h in (0, H // 3, 2 * H // 3, H - 1):
            picks.add((b, h, i_long))
    # rows that cross a ring refill right after a skipped block
    trig = np.argwhere(_refill_after_skip(gc, rec))
    for r in rng.permutation(len(trig))[:6]:
        picks.add(tuple(int(v) for v in trig[r]))
    # long rows on which the skip fired
    long_skip = np.argwhere((gc > 128) & (stats[..., 1] > 0))
    for r in rng.permutation(len(long_skip))[:6]:
        picks.add(tuple(int(v) for v in long_skip[r]))
    # any rows
    live = np.argwhere(gc > 0)
    for r in rng.permutation(len(live))[:4]:
        picks.add(tuple(int(v) for v in live[r]))
    return sorted(picks), len(trig), len(long_skip)


def _ascending(m):
    """The same kept sets with every row in ascending block order, pages
    looked up again (the remapping ablation's walk without the HRM-first
    order); built by sorting on the device, not by the oracle."""
    big = torch.iinfo(torch.int32).max
    blocks = torch.where(m.blocks < 0, torch.full_like(m.blocks, big), m.blocks)
    blocks = torch.sort(blocks, dim=-1).values
    blocks = torch.where(blocks == big, torch.full_like(blocks, -1), blocks).contiguous()
    # one page per block on these cases: the page of a block is found where
    # the original row lists it
    order = torch.argsort(torch.where(m.blocks < 0, torch.full_like(m.blocks, big), m.blocks),
                          dim=-1)
    pages = torch.gather(m.pages, -1, order)
    pages = torch.where(blocks < 0, torch.full_like(pages, -1), pages).contiguous()
    return bk.OrderedMask(blocks=blocks, pages=pages, counts=m.counts, hrm_counts=None,
                          capacity=m.capacity)


LONG_SKIP_CASES = [
    ("remap32k", {}, 1.0, 2.0, "kap"),
    ("remap32k", {}, 1.0, 6.0, "kap"),
    ("remap32k", {}, 0.3, 2.0, "kap"),
    ("remap32k", {}, 0.3, 6.0, "kap"),
    ("remap32k", {}, 1.0, 2.0, "ascending"),
    ("remap32k", {}, 1.0, 4.0, "ascending"),
    ("remap32k", {"kv_block": 128}, 1.0, 4.0, "kap"),
    ("remap128k", {}, 0.1, 8.0, "kap"),
]


@pytest.mark.parametrize("case", LONG_SKIP_CASES,
                         ids=[f"{n}{'-kv128' if kw else ''}-b{b}-t{t}-{o}"
                              for n, kw, b, t, o in LONG_SKIP_CASES])
def test_long_tile_skip_parity(case):
    name, kw, budget, tau, order = case
    w = ci.get(name).with_(**kw) if kw else ci.get(name)
    print(f"[case] long-tile skip {name} {kw} budget={budget} tau={tau} {order}: inputs",
          flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    print(f"[case] long-tile skip {name} {kw} budget={budget} tau={tau} {order}: GPU layer",
          flush=True)
    m = bk.proxy_ordered_mask(prob, q, k, budget)
    if order == "ascending":
        assert w.block == w.page_size
        m = _ascending(m)
    r = bk.osk_prefill(prob, q, k, v, m, tau)
    torch.cuda.synchronize()
    gb, gc = _np(m.blocks), _np(m.counts)
    out, lse, rec, stats = _np(r.out), _np(r.lse), _np(r.skip_record), _np(r.row_stats)
    del m, r, q, k, v
    assert np.all(np.isfinite(out))
    assert np.array_equal(stats[..., 0], gc)
    long_rows = gc > 128
    assert long_rows.any(), "no tile visits more than 128 blocks"
    assert int(stats[..., 1][long_rows].sum()) > 0, "the skip never fires on a long tile"
    picks, n_trig, n_long_skip = _long_tile_picks(w, gc, rec, stats, seed=w.seed + 7)
    lens = np.diff(x.cu_seqlens)
    grp = w.num_q_heads // w.num_kv_heads
    so, sl = ErrStats(), ErrStats()
    near = skipped = slots = 0
    cache = {}
    print(f"[case] long-tile skip {name}: oracle on {len(picks)} tiles", flush=True)
    for (b, h, i) in picks:
        s0, L = int(x.cu_seqlens[b]), int(lens[b])
        if b not in cache:
            cache = {b: (materialise(x.k_pool, x.page_table[b], L, w.page_size),
                         materialise(x.v_pool, x.page_table[b], L, w.page_size))}
        kk, vv = cache[b]
        g = h // grp
        rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
        qr = x.q[s0 + rows, h].astype(np.float64)
        cnt = int(gc[b, h, i])
        bl = gb[b, h, i, :cnt]
        res = oosk.osk_tile_closed_form(qr, rows, kk[:, g], vv[:, g], bl, tau,
                                        w.softmax_scale, w.block)
        near += check_osk_tile(out[s0 + rows, h], lse[h, s0 + rows], rec[b, h, i], res, qr,
                               rows, kk[:, g], vv[:, g], bl, w.softmax_scale, w.block, so, sl)
        assert stats[b, h, i, 1] == int(rec[b, h, i, :cnt].sum())
        skipped += int(rec[b, h, i, :cnt].sum())
        slots += cnt
    if order == "ascending":
        for (b, h, i) in picks:
            row = gb[b, h, i, :gc[b, h, i]]
            assert np.all(np.diff(row) > 0)
    report(f"long-tile skip {name}{'-kv128' if kw else ''} b={budget} tau={tau} {order}",
           tiles=len(picks), longest=int(gc.max()), refill_after_skip_rows=n_trig,
           long_rows_with_skips=n_long_skip, sampled_skipped=skipped, sampled_slots=slots,
           osk_near_threshold=near, layer_skip_ratio=round(
               float(stats[..., 1].sum()) / max(float(stats[..., 0].sum()), 1.0), 4))
    so.assert_ok(label=f"long-tile {name} osk out")
    sl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label=f"long-tile {name} osk lse")


def test_llama128k_every_block_ascending_equals_dense_bitwise():
    """The benchmark layer (llama128k) with every causal block of every tile
    in ascending order and the skip off: the ordered kernel then visits what
    the dense kernel visits, in the same order, with the same arithmetic, and
    the two agree bit for bit on every output and LSE value (1.07e9 + 4.2e6)."""
    w = ci.get("llama128k")
    print("[case] llama128k every block ascending vs dense: inputs", flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    L = int(x.cu_seqlens[1])
    nqb = (L + w.q_block - 1) // w.q_block
    C = (L + w.page_size - 1) // w.page_size
    n_i = (torch.minimum((torch.arange(nqb, device=DEV) + 1) * w.q_block,
                         torch.tensor(L, device=DEV)) - 1) // w.page_size + 1
    ar = torch.arange(C, device=DEV, dtype=torch.int32)
    valid = ar[None, :] < n_i[:, None]                              # [nqb][C]
    blocks = torch.where(valid, ar[None, :], torch.tensor(-1, device=DEV, dtype=torch.int32))
    pt = torch.from_numpy(x.page_table[0].astype(np.int32)).to(DEV)
    pages = torch.where(valid, pt[ar.long()][None, :], torch.tensor(-1, device=DEV,
                                                                    dtype=torch.int32))
    shape = (1, w.num_q_heads, nqb, C)
    mask = bk.OrderedMask(blocks=blocks[None, None].expand(shape).contiguous(),
                          pages=pages[None, None].expand(shape).contiguous(),
                          counts=n_i.to(torch.int32)[None, None].expand(shape[:3]).contiguous(),
                          hrm_counts=None, capacity=C)
    print("[case] llama128k every block ascending vs dense: GPU layer", flush=True)
    o = bk.osk_prefill(prob, q, k, v, mask, -1.0)
    d = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    assert int(o.row_stats[..., 1].sum()) == 0
    assert bool(torch.isfinite(d.out.float()).all())
    same_out = torch.equal(o.out, d.out)
    same_lse = torch.equal(o.lse, d.lse)
    report("llama128k ascending = dense", out_equal=same_out, lse_equal=same_lse,
           slots=int(n_i.sum()) * w.num_q_heads)
    assert same_out and same_lse


def test_stress_full_budget_skip_off_equals_dense():
    """The stress batch (16K + 48K + 96K + 128K in one pool) at a 100% stage-1
    budget with the in-kernel skip off (tau < 0, Delta = -1 of App. D.1): the
    OSK visits every causal block in the proxy's order and must give dense
    attention; compared with the dense kernel on every row and with the
    oracle on sampled tiles."""
    w = ci.get("stress")
    print("[case] stress beta=1 skip off: inputs", flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    print("[case] stress beta=1 skip off: GPU layer", flush=True)
    m = bk.proxy_ordered_mask(prob, q, k, 1.0)
    r = bk.osk_prefill(prob, q, k, v, m, -1.0)
    d = bk.dense_prefill(prob, q, k, v)
    torch.cuda.synchronize()
    gc, stats = _np(m.counts), _np(r.row_stats)
    lens = np.diff(x.cu_seqlens)
    for b in range(w.batch):
        nqb = (int(lens[b]) + w.q_block - 1) // w.q_block
        n_i = (np.minimum((np.arange(nqb) + 1) * w.q_block, lens[b]) - 1) // w.page_size + 1
        assert np.all(gc[b, :, :nqb] == n_i[None, :])
    assert int(stats[..., 1].sum()) == 0
    # every row: OSK against the dense kernel (a different visiting order),
    # reduced on the device (1.2e9 elements).  Each of the two bf16 results is
    # held to MAX_ABS / MEAN_ABS of the exact value (the sampled oracle check
    # below, and the dense kernel's own parity tests), so their difference is
    # bounded by twice that; one bf16 ulp of an output in [4, 8) is already
    # 2^-5.
    diff = (r.out.float() - d.out.float()).abs()
    assert bool(torch.isfinite(diff).all())
    mx, mean = float(diff.max()), float(diff.double().mean())
    del diff
    print(f"[parity] stress beta=1 osk vs dense kernel: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= 2 * MAX_ABS and mean <= 2 * MEAN_ABS, (mx, mean)
    out, lse = _np(r.out), _np(r.lse)
    del m, r, d, q, k, v
    picks = _sample(w, x, 10, seed=w.seed + 3)
    grp = w.num_q_heads // w.num_kv_heads
    so, sl = ErrStats(), ErrStats()
    cache = {}
    for (b, h, i) in picks:
        s0, L = int(x.cu_seqlens[b]), int(lens[b])
        if b not in cache:
            cache = {b: (materialise(x.k_pool, x.page_table[b], L, w.page_size),
                         materialise(x.v_pool, x.page_table[b], L, w.page_size))}
        kk, vv = cache[b]
        rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
        o, ls = odense.attention_rows(x.q[s0 + rows, h].astype(np.float64), rows,
                                      kk[:, h // grp], vv[:, h // grp], w.softmax_scale)
        so.add(out[s0 + rows, h], o)
        sl.add(lse[h, s0 + rows], ls)
    report("stress beta=1 skip off vs dense", tiles=len(picks),
           visited=int(stats[..., 0].sum()), kernel_max_abs=f"{mx:.2e}",
           kernel_mean_abs=f"{mean:.2e}")
    so.assert_ok(label="stress beta=1 osk vs oracle dense")
    sl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="stress beta=1 osk lse")


# The longest sequence the ABI accepts (2^20 tokens: 16384 key blocks, the
# size of the kernel's per-tile skip bitmap), beyond the proxy's 2048-block
# range, with masks built on the host.  Band-structured input (the remap128k
# pattern) so that the in-kernel skip fires on mixed-order walks.
MAXLEN = ci.get("remap128k").with_(name="max1m", seqlens=(1 << 20,), num_q_heads=2,
                                   num_kv_heads=1, seed=21)


def _max_len_mask(w, x, seed):
    """Ordered mask rows for every (head, tile): the diagonal block then five
    distinct earlier blocks in a seeded order; three long rows: every causal
    block of the last tile of head 0 shuffled (16384 slots, the slot ring
    refilled 256 times), 4096 of the 8192 blocks of a middle tile of head 1
    shuffled after its diagonal block, and every block of an early tile of
    head 0 in ascending order."""
    rng = np.random.default_rng(seed)
    L = int(x.seqlens[0])
    nqb = (L + w.q_block - 1) // w.q_block
    n_of = lambda i: (min((i + 1) * w.q_block, L) - 1) // w.block + 1  # noqa: E731
    cap = n_of(nqb - 1)
    long_rows = {}
    i0 = nqb - 1
    long_rows[(0, i0)] = rng.permutation(n_of(i0))
    i1 = nqb // 2 - 1
    n1 = n_of(i1)
    long_rows[(1, i1)] = np.concatenate([[n1 - 1], rng.choice(n1 - 1, size=4095, replace=False)])
    i2 = nqb // 4 - 1
    long_rows[(0, i2)] = np.arange(n_of(i2))
    blocks = np.full((1, w.num_q_heads, nqb, cap), -1, dtype=np.int32)
    counts = np.zeros((1, w.num_q_heads, nqb), dtype=np.int32)
    for h in range(w.num_q_heads):
        for i in range(nqb):
            n = n_of(i)
            if (h, i) in long_rows:
                row = long_rows[(h, i)]
            else:
                k = min(n, 6)
                row = np.concatenate([[n - 1], rng.choice(n - 1, size=k - 1, replace=False)])
            blocks[0, h, i, :len(row)] = row
            counts[0, h, i] = len(row)
    pt = x.page_table[0]
    pages = np.where(blocks >= 0, pt[np.maximum(blocks, 0)], -1).astype(np.int32)
    return blocks, pages, counts, cap, sorted(long_rows)


def test_osk_max_seqlen_host_mask():
    w = MAXLEN
    print("[case] 2^20-token sequence, host masks: inputs", flush=True)
    x = ci.make(w).bf16_rounded()
    prob, q, k, v = upload(x, DEV)
    blocks, pages, counts, cap, long_rows = _max_len_mask(w, x, seed=w.seed + 1)
    mask = bk.OrderedMask(blocks=torch.from_numpy(blocks).to(DEV),
                          pages=torch.from_numpy(pages).to(DEV),
                          counts=torch.from_numpy(counts).to(DEV), hrm_counts=None, capacity=cap)
    print(f"[case] 2^20-token sequence: GPU, skip off and tau 8 (capacity {cap})", flush=True)
    r_off = bk.osk_prefill(prob, q, k, v, mask, -1.0)
    r_on = bk.osk_prefill(prob, q, k, v, mask, w.tau)
    torch.cuda.synchronize()
    res = {}
    for name, r in (("off", r_off), ("on", r_on)):
        res[name] = (_np(r.out), _np(r.lse), _np(r.skip_record), _np(r.row_stats))
    del mask, r_off, r_on, q, k, v
    for name, (out, lse, rec, stats) in res.items():
        assert np.all(np.isfinite(out)), name
        assert np.array_equal(stats[..., 0], counts), name
    assert int(res["off"][3][..., 1].sum()) == 0
    n_skip = int(res["on"][3][..., 1].sum())
    assert n_skip > 0, "the skip never fires"
    L = int(x.seqlens[0])
    kk = materialise(x.k_pool, x.page_table[0], L, w.page_size)[:, 0]
    vv = materialise(x.v_pool, x.page_table[0], L, w.page_size)[:, 0]
    rng = np.random.default_rng(w.seed + 2)
    nqb = blocks.shape[2]
    short = [(int(rng.integers(2)), int(rng.integers(nqb))) for _ in range(6)]
    print(f"[case] 2^20-token sequence: oracle on {len(long_rows) + len(short)} tiles",
          flush=True)
    so_off, sl_off, so_on, sl_on = ErrStats(), ErrStats(), ErrStats(), ErrStats()
    near = 0
    for (h, i) in long_rows + short:
        rows = np.arange(i * w.q_block, min((i + 1) * w.q_block, L))
        qr = x.q[rows, h].astype(np.float64)
        cnt = int(counts[0, h, i])
        bl = blocks[0, h, i, :cnt]
        # skip off: attention over the keys of the listed blocks
        key_ok = np.zeros(L, dtype=bool)
        for j in bl:
            key_ok[j * w.block:min((j + 1) * w.block, L)] = True
        o, ls = odense.attention_rows(qr, rows, kk, vv, w.softmax_scale, key_ok=key_ok)
        out, lse, rec, _ = res["off"]
        so_off.add(out[rows, h], o)
        sl_off.add(lse[h, rows], ls)
        # tau 8: the closed form of the skip (the 16384-slot row only above)
        if cnt > 8192:
            continue
        tr = oosk.osk_tile_closed_form(qr, rows, kk, vv, bl, w.tau, w.softmax_scale, w.block)
        out, lse, rec, _ = res["on"]
        near += check_osk_tile(out[rows, h], lse[h, rows], rec[0, h, i], tr, qr, rows, kk, vv,
                               bl, w.softmax_scale, w.block, so_on, sl_on)
    report("2^20-token sequence, host masks", tiles=len(long_rows) + len(short),
           capacity=cap, longest=int(counts.max()), layer_skipped=n_skip,
           osk_near_threshold=near)
    so_off.assert_ok(label="2^20 skip off out")
    sl_off.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="2^20 skip off lse")
    so_on.assert_ok(label="2^20 tau 8 out")
    sl_on.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="2^20 tau 8 lse")
