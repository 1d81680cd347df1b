"""Pins for the dense causal attention oracle (CPU, float64).

Dense attention is a textbook definition (CoSA (paperpeel) §3.1 heading; the
full-attention baseline of §5.1).  It is pinned to: torch's
scaled_dot_product_attention in float64 on the CPU (a library routine), a
pure-Python brute force on tiny inputs, and two closed forms (zero queries give
the running mean of the values; logsumexp of the exact logits).
"""
import math

import numpy as np
import pytest
import torch

from oracle.dense import attention_rows, dense_causal_attention
from oracle.paging import materialise

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_dense_matches_torch_sdpa_fp64_gqa():
    L, Hq, Hkv, D = 203, 4, 2, 16
    q, k, v = _rand(1, L, Hq, D), _rand(2, L, Hkv, D), _rand(3, L, Hkv, D)
    scale = 1 / math.sqrt(D)
    out, lse = dense_causal_attention(q, k, v, scale, row_chunk=64)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]               # [1][Hq][L][D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    # lse against an independent logsumexp of the causal logits
    from scipy.special import logsumexp
    for h in range(Hq):
        s = scale * q[:, h] @ k[:, h // 2].T
        s[np.triu_indices(L, 1)] = -np.inf
        assert np.max(np.abs(lse[h] - logsumexp(s, axis=1))) < 1e-12


def test_dense_pure_python_brute_force():
    L, D = 7, 3
    q, k, v = _rand(4, L, 1, D), _rand(5, L, 1, D), _rand(6, L, 1, D)
    scale = 0.7
    out, lse = dense_causal_attention(q, k, v, scale)
    for t in range(L):
        logits = [scale * sum(q[t, 0, d] * k[u, 0, d] for d in range(D)) for u in range(t + 1)]
        mx = max(logits)
        ex = [math.exp(x - mx) for x in logits]
        z = sum(ex)
        for d in range(D):
            ref = sum(ex[u] * v[u, 0, d] for u in range(t + 1)) / z
            assert abs(out[t, 0, d] - ref) < 1e-13
        assert abs(lse[0, t] - (mx + math.log(z))) < 1e-13


def test_zero_queries_give_running_mean_of_values():
    # closed form: q = 0 makes every allowed logit 0, so the softmax is uniform
    # over keys 0..t and the output is the running mean of the values.
    L, D = 50, 8
    q = np.zeros((L, 2, D))
    k, v = _rand(7, L, 1, D), _rand(8, L, 1, D)
    out, lse = dense_causal_attention(q, k, v, 0.3)
    run_mean = np.cumsum(v[:, 0], axis=0) / np.arange(1, L + 1)[:, None]
    assert np.max(np.abs(out[:, 0] - run_mean)) < 1e-13
    assert np.max(np.abs(out[:, 1] - run_mean)) < 1e-13
    assert np.max(np.abs(lse[0] - np.log(np.arange(1, L + 1)))) < 1e-13


def test_row_without_keys_gives_zero_and_neg_inf():
    k, v = _rand(9, 4, 3), _rand(10, 4, 3)
    out, lse = attention_rows(_rand(11, 2, 3), np.array([1, 3]), k, v, 1.0,
                              key_ok=np.array([False, False, True, True]))
    assert np.all(out[0] == 0) and np.isneginf(lse[0])
    assert np.isfinite(lse[1])


def test_materialise_follows_page_table():
    # hand-built pool: token t of head hh has value 1000*hh + t in every dim
    page, H, D, L = 4, 2, 3, 10
    table = np.array([5, 0, 3, -1], dtype=np.int32)
    pool = np.full((6, H, page, D), np.nan)
    for t in range(L):
        for hh in range(H):
            pool[table[t // page], hh, t % page, :] = 1000 * hh + t
    x = materialise(pool, table, L, page)
    assert x.shape == (L, H, D)
    for t in range(L):
        for hh in range(H):
            assert np.all(x[t, hh] == 1000 * hh + t)
