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

from .parity import ErrStats, check_kap_row, check_osk_tile, upload

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
    m = bk.proxy_ordered_mask(prob, q, k, w.budget)
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
    # sampled oracle checks
    grp = w.num_q_heads // w.num_kv_heads
    kap_exact = kap_tie = 0
    so, sl, do, dl = ErrStats(), ErrStats(), ErrStats(), ErrStats()
    near = 0
    cache = {}
    picks = _sample(w, x, n_samples, seed=w.seed)
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
    print(f"[parity] {name}: KAP exact={kap_exact} near-tie={kap_tie}; OSK near-threshold "
          f"slots={near}; layer skipped={int(stats[..., 1].sum())} of {int(stats[..., 0].sum())}")
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
    print(f"[parity] shared-kv llama128k: KAP rows exact={exact} of {len(picks)}; "
          f"near-threshold slots={near}")
    so.assert_ok(label="shared-kv osk out")
    sl.assert_ok(max_abs=1e-3, mean_abs=1e-4, label="shared-kv osk lse")
    assert exact >= len(picks) // 2
