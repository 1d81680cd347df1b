"""The C-ABI library loads and behaves on the host without a GPU.

Checks that ``libcosa.so`` exports every function ``include/cosa.h``
declares, and exercises the host-side paths that return before any HIP call:
argument validation with its status codes, capacity and workspace sizing
(compared with the oracle's own budget rule), and the host page-table check.
No kernel is launched here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_long_kap_amd import _lib
from oracle import kap as okap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cosa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_long_kap_amd.build import build_library
        build_library()
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cosa_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.cosa_abi_version() == 1


def _problem(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, q_block=128,
                kv_block=64, page_size=64, max_seqlen=131072, max_pages_per_seq=2048,
                num_pages=2112, total_q=131072, softmax_scale=128 ** -0.5,
                cu_seqlens=0x1000, page_table=0x2000)
    base.update(kw)
    return _lib.CosaProblem(**base)


BAD = [
    (dict(batch=0), _lib.COSA_ERR_INVALID_ARG),
    (dict(num_q_heads=30), _lib.COSA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), _lib.COSA_ERR_INVALID_ARG),
    (dict(head_dim=96), _lib.COSA_ERR_UNSUPPORTED),
    (dict(q_block=32), _lib.COSA_ERR_UNSUPPORTED),
    (dict(page_size=16, kv_block=16), _lib.COSA_ERR_UNSUPPORTED),
    (dict(kv_block=192), _lib.COSA_ERR_UNSUPPORTED),
    (dict(kv_block=32), _lib.COSA_ERR_UNSUPPORTED),
    # two-page logical blocks need page-table rows covering whole blocks
    (dict(kv_block=128, max_seqlen=130945, total_q=130945, max_pages_per_seq=2047),
     _lib.COSA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), _lib.COSA_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=100), _lib.COSA_ERR_INVALID_ARG),
    (dict(num_pages=0), _lib.COSA_ERR_INVALID_ARG),
    (dict(total_q=131073), _lib.COSA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), _lib.COSA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), _lib.COSA_ERR_INVALID_ARG),
    (dict(cu_seqlens=None), _lib.COSA_ERR_INVALID_ARG),
    (dict(page_table=None), _lib.COSA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("case", range(len(BAD)))
def test_validation_status_codes(lib, case):
    kw, code = BAD[case]
    p = _problem(**kw)
    assert lib.cosa_validate_problem(ctypes.byref(p)) == code
    assert lib.cosa_last_error().decode() != ""
    # every entry point rejects it before launching anything
    assert lib.cosa_dense_prefill(ctypes.byref(p), 1, 1, 1, 1, None, None) == code
    assert lib.cosa_osk_prefill(ctypes.byref(p), 1, 1, 1, 1, 1, 1, 5, 1.0, 1, None, None, None,
                                None) == code
    assert lib.cosa_proxy_ordered_mask(ctypes.byref(p), 1, 1, 0.1, 1, 1, 1, None, None, None,
                                       1000, 1, 1 << 40, None) == code
    assert lib.cosa_kap_workspace_size(ctypes.byref(p)) == 0


def test_null_problem_and_status_strings(lib):
    assert lib.cosa_validate_problem(None) == _lib.COSA_ERR_INVALID_ARG
    for s, name in [(0, "COSA_OK"), (-1, "COSA_ERR_INVALID_ARG"), (-2, "COSA_ERR_UNSUPPORTED"),
                    (-3, "COSA_ERR_WORKSPACE"), (-4, "COSA_ERR_HIP")]:
        assert lib.cosa_status_string(s).decode() == name


@pytest.mark.parametrize("seqlen,budget", [(131072, 0.1), (131072, 0.05), (131072, 0.3),
                                           (32768, 0.2), (2048, 0.5), (100, 1.0), (1, 0.01),
                                           (131072, 1e-9)])
def test_capacity_and_tiles_follow_the_budget_rule(lib, seqlen, budget):
    p = _problem(max_seqlen=seqlen, total_q=seqlen)
    beta = max(okap.budget_ppm(budget), 1)
    assert lib.cosa_mask_capacity(ctypes.byref(p), budget) == \
        okap.mask_capacity(seqlen, 64, beta)
    assert lib.cosa_num_q_tiles(ctypes.byref(p)) == -(-seqlen // 128)
    nkb = -(-seqlen // 64)
    # bf16 hi and lo planes of the pooled keys, blocks padded to a multiple of 32
    assert lib.cosa_kap_workspace_size(ctypes.byref(p)) == 8 * 128 * (-(-nkb // 32) * 32) * 4
    for bad in (0.0, -0.1, 1.5, float("nan")):
        assert lib.cosa_mask_capacity(ctypes.byref(p), bad) == _lib.COSA_ERR_INVALID_ARG


def test_entry_points_reject_bad_buffers(lib):
    p = _problem()
    pr = ctypes.byref(p)
    E = _lib.COSA_ERR_INVALID_ARG
    assert lib.cosa_dense_prefill(pr, None, 1, 1, 1, None, None) == E
    assert lib.cosa_dense_prefill(pr, 1, 1, 1, None, None, None) == E
    assert lib.cosa_osk_prefill(pr, 1, 1, 1, None, 1, 1, 5, 1.0, 1, None, None, None, None) == E
    assert lib.cosa_osk_prefill(pr, 1, 1, 1, 1, 1, 1, 0, 1.0, 1, None, None, None, None) == E
    assert lib.cosa_osk_prefill(pr, 1, 1, 1, 1, 1, 1, 5, float("nan"), 1, None, None, None,
                                None) == E
    cap = lib.cosa_mask_capacity(pr, 0.1)
    ws = lib.cosa_kap_workspace_size(pr)
    assert lib.cosa_proxy_ordered_mask(pr, 1, 1, 0.1, 1, 1, 1, None, None, None, cap - 1, 1, ws,
                                       None) == E
    assert lib.cosa_proxy_ordered_mask(pr, 1, 1, 0.1, 1, 1, 1, None, None, None, cap, 1, ws - 1,
                                       None) == _lib.COSA_ERR_WORKSPACE
    assert lib.cosa_proxy_ordered_mask(pr, 1, 1, 0.1, 1, 1, 1, None, None, None, cap, None, ws,
                                       None) == _lib.COSA_ERR_WORKSPACE
    assert lib.cosa_proxy_ordered_mask(pr, 1, 1, 0.0, 1, 1, 1, None, None, None, cap, 1, ws,
                                       None) == E
    # Top-p outside (0, 1], a bad cap and a short capacity are refused before any launch
    for bad_p in (0.0, -0.5, 1.01, float("nan")):
        assert lib.cosa_proxy_ordered_mask_top_p(pr, 1, 1, bad_p, 0.1, 1, 1, 1, None, None, None,
                                                 cap, 1, ws, None) == E
    assert lib.cosa_proxy_ordered_mask_top_p(pr, 1, 1, 0.9, 0.0, 1, 1, 1, None, None, None, cap,
                                             1, ws, None) == E
    assert lib.cosa_proxy_ordered_mask_top_p(pr, 1, 1, 0.9, 0.1, 1, 1, 1, None, None, None,
                                             cap - 1, 1, ws, None) == E
    # Delta must be finite; the mask arrays are required
    for bad_d in (float("nan"), float("inf"), float("-inf")):
        assert lib.cosa_osk_prefill_delta(pr, 1, 1, 1, 1, 1, 1, 5, bad_d, 1, None, None, None,
                                          None) == E
    assert lib.cosa_osk_prefill_delta(pr, 1, 1, 1, None, 1, 1, 5, 200.0, 1, None, None, None,
                                      None) == E
    # the fused call checks both halves' arguments before any launch
    def fused(budget=0.1, tau=8.0, v=1, capacity=cap, wsb=ws, out=1, stream=None, aux=None):
        return lib.cosa_sparse_prefill(pr, 1, 1, v, budget, tau, 1, 1, 1, None, capacity, 1, wsb,
                                       out, None, None, None, stream, aux)
    assert fused(budget=0.0) == E
    assert fused(capacity=cap - 1) == E
    assert fused(wsb=ws - 1) == _lib.COSA_ERR_WORKSPACE
    assert fused(v=None) == E
    assert fused(out=None) == E
    assert fused(tau=float("nan")) == E
    assert fused(stream=7, aux=7) == E
    # the proxy handles at most 2048 key blocks per sequence
    big = _problem(max_seqlen=131073, max_pages_per_seq=2049, total_q=131073)
    assert lib.cosa_proxy_ordered_mask(ctypes.byref(big), 1, 1, 0.1, 1, 1, 1, None, None, None,
                                       10 ** 6, 1, 1 << 40, None) == _lib.COSA_ERR_UNSUPPORTED


def test_host_page_table_check(lib):
    p = _problem(batch=2, max_seqlen=200, max_pages_per_seq=4, num_pages=8, total_q=330)
    cu = np.array([0, 200, 330], dtype=np.int32)
    pt = np.array([[3, 1, 0, 7], [2, 5, 6, -1]], dtype=np.int32)   # seq 1 uses 3 pages
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.cosa_check_page_table_host(ctypes.byref(p), vp(cu), vp(pt)) == 0
    bad = pt.copy()
    bad[1, 2] = 8
    assert lib.cosa_check_page_table_host(ctypes.byref(p), vp(cu), vp(bad)) == -1
    bad = pt.copy()
    bad[0, 0] = -1
    assert lib.cosa_check_page_table_host(ctypes.byref(p), vp(cu), vp(bad)) == -1
    cu_bad = np.array([0, 201, 330], dtype=np.int32)
    assert lib.cosa_check_page_table_host(ctypes.byref(p), vp(cu_bad), vp(pt)) == -1
    cu_bad = np.array([0, 200, 331], dtype=np.int32)
    assert lib.cosa_check_page_table_host(ctypes.byref(p), vp(cu_bad), vp(pt)) == -1
    assert lib.cosa_check_page_table_host(ctypes.byref(p), None, vp(pt)) == -1


def test_no_alloc_proxy_rejects_before_any_hip_call(lib):
    """cosa_proxy_ordered_mask_no_alloc checks its arguments and the size of
    the static workspace on the host, before it looks up the device."""
    p = _problem()
    pr = ctypes.byref(p)
    cap = lib.cosa_mask_capacity(pr, 0.1)
    E = _lib.COSA_ERR_INVALID_ARG
    assert lib.cosa_proxy_ordered_mask_no_alloc(pr, None, 1, 0.1, 1, 1, 1, None, None, None,
                                                cap, None) == E
    assert lib.cosa_proxy_ordered_mask_no_alloc(pr, 1, 1, 0.1, 1, 1, 1, None, None, None,
                                                cap - 1, None) == E
    assert lib.cosa_proxy_ordered_mask_no_alloc(pr, 1, 1, 1.5, 1, 1, 1, None, None, None,
                                                cap, None) == E
    # four 128K sequences with 8 KV heads fit the 32 MiB array exactly, five do not
    fits = _problem(batch=4, total_q=4 * 131072)
    assert lib.cosa_kap_workspace_size(ctypes.byref(fits)) == _lib.NO_ALLOC_SCRATCH_BYTES
    big = _problem(batch=5, total_q=5 * 131072)
    assert lib.cosa_kap_workspace_size(ctypes.byref(big)) > _lib.NO_ALLOC_SCRATCH_BYTES
    assert lib.cosa_proxy_ordered_mask_no_alloc(ctypes.byref(big), 1, 1, 0.1, 1, 1, 1, None,
                                                None, None, cap, None) == \
        _lib.COSA_ERR_WORKSPACE
    assert "COSA_NO_ALLOC_SCRATCH_BYTES" in lib.cosa_last_error().decode()
    # the header states the same size
    assert re.search(r"#define COSA_NO_ALLOC_SCRATCH_BYTES \(32u << 20\)", open(HEADER).read())
