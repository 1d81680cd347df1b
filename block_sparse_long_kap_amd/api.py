"""Python binding of the C ABI: tensors in, tensors out, nothing computed here.

Every function checks shapes/dtypes/devices, allocates outputs with torch on
the inputs' device (torch is used for device memory and streams only), and
calls the matching ``cosa_*`` entry point on the current HIP stream.  All
arithmetic happens in the gfx950 kernels of ``libcosa.so``.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device, ndim=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class Problem:
    """One layer's prefill problem; mirrors ``cosa_problem``.

    ``cu_seqlens`` (int32 [B+1]) and ``page_table`` (int32 [B][max_pages]) are
    device tensors; ``max_seqlen`` and ``total_q`` are host integers.
    """
    cu_seqlens: torch.Tensor
    page_table: torch.Tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_seqlen: int
    total_q: int
    num_pages: int
    q_block: int = 128
    page_size: int = 64
    softmax_scale: Optional[float] = None
    kv_block: Optional[int] = None   # logical key block; default one page

    def __post_init__(self):
        if self.softmax_scale is None:
            self.softmax_scale = 1.0 / math.sqrt(self.head_dim)
        if self.kv_block is None:
            self.kv_block = self.page_size
        dev = self.cu_seqlens.device
        _need(self.cu_seqlens, "cu_seqlens", torch.int32, dev, ndim=1)
        _need(self.page_table, "page_table", torch.int32, dev, ndim=2)
        self._c = _lib.CosaProblem(
            batch=self.cu_seqlens.numel() - 1, num_q_heads=self.num_q_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, q_block=self.q_block,
            kv_block=self.kv_block, page_size=self.page_size, max_seqlen=self.max_seqlen,
            max_pages_per_seq=self.page_table.shape[1], num_pages=self.num_pages,
            total_q=self.total_q, softmax_scale=self.softmax_scale,
            cu_seqlens=self.cu_seqlens.data_ptr(), page_table=self.page_table.data_ptr())

    @property
    def device(self) -> torch.device:
        return self.cu_seqlens.device

    @property
    def batch(self) -> int:
        return self.cu_seqlens.numel() - 1

    @property
    def c(self) -> _lib.CosaProblem:
        return self._c

    def ref(self):
        return ctypes.byref(self._c)

    def num_q_tiles(self) -> int:
        n = _lib.load().cosa_num_q_tiles(self.ref())
        if n < 0:
            _lib.check(int(n), "cosa_num_q_tiles")
        return int(n)

    def mask_capacity(self, budget: float) -> int:
        n = _lib.load().cosa_mask_capacity(self.ref(), ctypes.c_float(budget))
        if n < 0:
            _lib.check(int(n), "cosa_mask_capacity")
        return int(n)

    def kap_workspace_size(self) -> int:
        return int(_lib.load().cosa_kap_workspace_size(self.ref()))

    def validate(self) -> None:
        _lib.check(_lib.load().cosa_validate_problem(self.ref()), "cosa_validate_problem")

    def check_host_tables(self, cu_host, table_host) -> None:
        """Validate host copies (numpy int32) of cu_seqlens and page_table."""
        import numpy as np
        cu = np.ascontiguousarray(cu_host, dtype=np.int32)
        pt = np.ascontiguousarray(table_host, dtype=np.int32)
        _lib.check(_lib.load().cosa_check_page_table_host(
            self.ref(), cu.ctypes.data_as(ctypes.c_void_p), pt.ctypes.data_as(ctypes.c_void_p)),
            "cosa_check_page_table_host")

    def _check_qkv(self, q, k_pool, v_pool=None):
        dev = self.device
        _need(q, "q", torch.bfloat16, dev, shape=(self.total_q, self.num_q_heads, self.head_dim))
        pool_shape = (self.num_pages, self.num_kv_heads, self.page_size, self.head_dim)
        _need(k_pool, "k_pool", torch.bfloat16, dev, shape=pool_shape)
        if v_pool is not None:
            _need(v_pool, "v_pool", torch.bfloat16, dev, shape=pool_shape)


@dataclass
class OrderedMask:
    blocks: torch.Tensor          # int32 [B][Hq][NQB][C]
    pages: torch.Tensor           # int32 [B][Hq][NQB][C]
    counts: torch.Tensor          # int32 [B][Hq][NQB]
    hrm_counts: Optional[torch.Tensor]
    capacity: int
    debug_w: Optional[torch.Tensor] = None     # fp32 [B][Hq][NQB][n_max]
    debug_hrm: Optional[torch.Tensor] = None   # uint8 [B][Hq][NQB][n_max]


class KapWorkspace:
    """Reusable device workspace for the proxy (pooled keys)."""

    def __init__(self, problem: Problem):
        self.nbytes = problem.kap_workspace_size()
        self.buf = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device=problem.device)


def _mask_buffers(problem: Problem, q, k_pool, budget, capacity, hrm_counts, debug, out,
                  shared_kv=False):
    problem._check_qkv(q, k_pool)
    dev = problem.device
    C = problem.mask_capacity(budget) if capacity is None else int(capacity)
    nqb = problem.num_q_tiles()
    rows = (problem.batch, problem.num_kv_heads if shared_kv else problem.num_q_heads, nqb)
    if out is None:
        ppb = problem.kv_block // problem.page_size
        out = OrderedMask(
            blocks=torch.empty(rows + (C,), dtype=torch.int32, device=dev),
            pages=torch.empty(rows + (C * ppb,), dtype=torch.int32, device=dev),
            counts=torch.empty(rows, dtype=torch.int32, device=dev),
            hrm_counts=torch.empty(rows, dtype=torch.int32, device=dev) if hrm_counts else None,
            capacity=C)
        if debug:
            n_max = -(-problem.max_seqlen // problem.kv_block)
            out.debug_w = torch.empty(rows + (n_max,), dtype=torch.float32, device=dev)
            out.debug_hrm = torch.empty(rows + (n_max,), dtype=torch.uint8, device=dev)
    return out


def proxy_ordered_mask(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor, budget: float,
                       *, capacity: Optional[int] = None, hrm_counts: bool = True,
                       debug: bool = False, workspace: Optional[KapWorkspace] = None,
                       out: Optional[OrderedMask] = None) -> OrderedMask:
    """KAP ordered mask (``cosa_proxy_ordered_mask``)."""
    lib = _lib.load()
    out = _mask_buffers(problem, q, k_pool, budget, capacity, hrm_counts, debug, out)
    ws = workspace if workspace is not None else KapWorkspace(problem)
    st = lib.cosa_proxy_ordered_mask(
        problem.ref(), _ptr(q), _ptr(k_pool), ctypes.c_float(budget), _ptr(out.blocks),
        _ptr(out.pages), _ptr(out.counts), _ptr(out.hrm_counts), _ptr(out.debug_w),
        _ptr(out.debug_hrm), out.capacity, _ptr(ws.buf), ws.nbytes, _stream(problem.device))
    _lib.check(st, "cosa_proxy_ordered_mask")
    return out


def proxy_ordered_mask_no_alloc(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                                budget: float, *, capacity: Optional[int] = None,
                                hrm_counts: bool = True, debug: bool = False,
                                out: Optional[OrderedMask] = None) -> OrderedMask:
    """KAP ordered mask with the library's static workspace
    (``cosa_proxy_ordered_mask_no_alloc``): pass ``out`` to allocate nothing
    on this side either."""
    lib = _lib.load()
    out = _mask_buffers(problem, q, k_pool, budget, capacity, hrm_counts, debug, out)
    st = lib.cosa_proxy_ordered_mask_no_alloc(
        problem.ref(), _ptr(q), _ptr(k_pool), ctypes.c_float(budget), _ptr(out.blocks),
        _ptr(out.pages), _ptr(out.counts), _ptr(out.hrm_counts), _ptr(out.debug_w),
        _ptr(out.debug_hrm), out.capacity, _stream(problem.device))
    _lib.check(st, "cosa_proxy_ordered_mask_no_alloc")
    return out


def proxy_ordered_mask_top_p(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                             top_p: float, budget: float = 1.0, *,
                             capacity: Optional[int] = None, hrm_counts: bool = True,
                             debug: bool = False, workspace: Optional[KapWorkspace] = None,
                             out: Optional[OrderedMask] = None) -> OrderedMask:
    """KAP ordered mask with stage-1 Top-p under a budget cap
    (``cosa_proxy_ordered_mask_top_p``)."""
    lib = _lib.load()
    out = _mask_buffers(problem, q, k_pool, budget, capacity, hrm_counts, debug, out)
    ws = workspace if workspace is not None else KapWorkspace(problem)
    st = lib.cosa_proxy_ordered_mask_top_p(
        problem.ref(), _ptr(q), _ptr(k_pool), ctypes.c_float(top_p), ctypes.c_float(budget),
        _ptr(out.blocks), _ptr(out.pages), _ptr(out.counts), _ptr(out.hrm_counts),
        _ptr(out.debug_w), _ptr(out.debug_hrm), out.capacity, _ptr(ws.buf), ws.nbytes,
        _stream(problem.device))
    _lib.check(st, "cosa_proxy_ordered_mask_top_p")
    return out


@dataclass
class PrefillOutput:
    out: torch.Tensor                      # bf16 [T][Hq][D]
    lse: Optional[torch.Tensor]            # fp32 [Hq][T]
    skip_record: Optional[torch.Tensor] = None   # uint8 [B][Hq][NQB][C]
    row_stats: Optional[torch.Tensor] = None     # int32 [B][Hq][NQB][2]


def _prefill_buffers(problem: Problem, q, k_pool, v_pool, mask, lse, record, out,
                     shared_kv=False):
    problem._check_qkv(q, k_pool, v_pool)
    dev = problem.device
    nqb = problem.num_q_tiles()
    rows = (problem.batch, problem.num_q_heads, nqb)
    mrows = (problem.batch, problem.num_kv_heads, nqb) if shared_kv else rows
    _need(mask.blocks, "mask.blocks", torch.int32, dev, shape=mrows + (mask.capacity,))
    ppb = problem.kv_block // problem.page_size
    _need(mask.pages, "mask.pages", torch.int32, dev, shape=mrows + (mask.capacity * ppb,))
    _need(mask.counts, "mask.counts", torch.int32, dev, shape=mrows)
    if out is None:
        out = PrefillOutput(
            out=torch.empty_like(q),
            lse=torch.empty((problem.num_q_heads, problem.total_q), dtype=torch.float32,
                            device=dev) if lse else None,
            skip_record=torch.zeros(rows + (mask.capacity,), dtype=torch.uint8, device=dev)
            if record else None,
            row_stats=torch.zeros(rows + (2,), dtype=torch.int32, device=dev) if record else None)
    return out


def osk_prefill(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                mask: OrderedMask, skip_tau: float, *, lse: bool = True, record: bool = True,
                out: Optional[PrefillOutput] = None) -> PrefillOutput:
    """Ordered-Skipping Kernel (``cosa_osk_prefill``); skip_tau < 0 disables the skip."""
    lib = _lib.load()
    out = _prefill_buffers(problem, q, k_pool, v_pool, mask, lse, record, out)
    st = lib.cosa_osk_prefill(problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                              _ptr(mask.blocks), _ptr(mask.pages), _ptr(mask.counts),
                              mask.capacity, ctypes.c_float(skip_tau), _ptr(out.out),
                              _ptr(out.lse), _ptr(out.skip_record), _ptr(out.row_stats),
                              _stream(problem.device))
    _lib.check(st, "cosa_osk_prefill")
    return out


def proxy_ordered_mask_shared_kv(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                                 budget: float, top_p: float = 1.0, *,
                                 capacity: Optional[int] = None, hrm_counts: bool = True,
                                 debug: bool = False, workspace: Optional[KapWorkspace] = None,
                                 out: Optional[OrderedMask] = None) -> OrderedMask:
    """KAP with one mask per KV head shared by its query heads
    (``cosa_proxy_ordered_mask_shared_kv``); arrays are [B][Hkv][NQB](...)."""
    lib = _lib.load()
    out = _mask_buffers(problem, q, k_pool, budget, capacity, hrm_counts, debug, out,
                        shared_kv=True)
    ws = workspace if workspace is not None else KapWorkspace(problem)
    st = lib.cosa_proxy_ordered_mask_shared_kv(
        problem.ref(), _ptr(q), _ptr(k_pool), ctypes.c_float(top_p), ctypes.c_float(budget),
        _ptr(out.blocks), _ptr(out.pages), _ptr(out.counts), _ptr(out.hrm_counts),
        _ptr(out.debug_w), _ptr(out.debug_hrm), out.capacity, _ptr(ws.buf), ws.nbytes,
        _stream(problem.device))
    _lib.check(st, "cosa_proxy_ordered_mask_shared_kv")
    return out


def osk_prefill_shared_kv(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                          v_pool: torch.Tensor, mask: OrderedMask, skip_tau: float, *,
                          lse: bool = True, record: bool = True,
                          out: Optional[PrefillOutput] = None) -> PrefillOutput:
    """Ordered-Skipping Kernel over per-KV-head masks (``cosa_osk_prefill_shared_kv``)."""
    lib = _lib.load()
    out = _prefill_buffers(problem, q, k_pool, v_pool, mask, lse, record, out, shared_kv=True)
    st = lib.cosa_osk_prefill_shared_kv(problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(mask.blocks), _ptr(mask.pages), _ptr(mask.counts),
                                        mask.capacity, ctypes.c_float(skip_tau), _ptr(out.out),
                                        _ptr(out.lse), _ptr(out.skip_record),
                                        _ptr(out.row_stats), _stream(problem.device))
    _lib.check(st, "cosa_osk_prefill_shared_kv")
    return out


def osk_prefill_delta(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, mask: OrderedMask, skip_delta: float, *,
                      lse: bool = True, record: bool = True,
                      out: Optional[PrefillOutput] = None) -> PrefillOutput:
    """Ordered-Skipping Kernel with the per-sequence threshold ln(L_b / Delta)
    (``cosa_osk_prefill_delta``); skip_delta <= 0 disables the skip."""
    lib = _lib.load()
    out = _prefill_buffers(problem, q, k_pool, v_pool, mask, lse, record, out)
    st = lib.cosa_osk_prefill_delta(problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(mask.blocks), _ptr(mask.pages), _ptr(mask.counts),
                                    mask.capacity, ctypes.c_float(skip_delta), _ptr(out.out),
                                    _ptr(out.lse), _ptr(out.skip_record), _ptr(out.row_stats),
                                    _stream(problem.device))
    _lib.check(st, "cosa_osk_prefill_delta")
    return out


def sparse_prefill(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   budget: float, skip_tau: float, *, aux_stream: Optional[torch.cuda.Stream] = None,
                   capacity: Optional[int] = None, hrm_counts: bool = True,
                   workspace: Optional[KapWorkspace] = None, mask: Optional[OrderedMask] = None,
                   lse: bool = True, record: bool = True,
                   out: Optional[PrefillOutput] = None):
    """KAP mask and OSK attention in one call (``cosa_sparse_prefill``); returns
    (mask, output).  With ``aux_stream`` the kernel of each chunk of KV groups
    runs there while the proxy of the next chunk runs on the current stream."""
    lib = _lib.load()
    mask = _mask_buffers(problem, q, k_pool, budget, capacity, hrm_counts, False, mask)
    ws = workspace if workspace is not None else KapWorkspace(problem)
    out = _prefill_buffers(problem, q, k_pool, v_pool, mask, lse, record, out)
    aux = None if aux_stream is None else ctypes.c_void_p(aux_stream.cuda_stream)
    st = lib.cosa_sparse_prefill(
        problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool), ctypes.c_float(budget),
        ctypes.c_float(skip_tau), _ptr(mask.blocks), _ptr(mask.pages), _ptr(mask.counts),
        _ptr(mask.hrm_counts), mask.capacity, _ptr(ws.buf), ws.nbytes, _ptr(out.out),
        _ptr(out.lse), _ptr(out.skip_record), _ptr(out.row_stats), _stream(problem.device), aux)
    _lib.check(st, "cosa_sparse_prefill")
    return mask, out


def dense_prefill(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  *, lse: bool = True, out: Optional[PrefillOutput] = None) -> PrefillOutput:
    """Dense causal prefill on the same kernel (``cosa_dense_prefill``)."""
    lib = _lib.load()
    problem._check_qkv(q, k_pool, v_pool)
    dev = problem.device
    if out is None:
        out = PrefillOutput(
            out=torch.empty_like(q),
            lse=torch.empty((problem.num_q_heads, problem.total_q), dtype=torch.float32,
                            device=dev) if lse else None)
    st = lib.cosa_dense_prefill(problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(out.out), _ptr(out.lse), _stream(dev))
    _lib.check(st, "cosa_dense_prefill")
    return out


def block_mask_prefill(problem: Problem, q: torch.Tensor, k_pool: torch.Tensor,
                       v_pool: torch.Tensor, block_mask: torch.Tensor, *, lse: bool = True,
                       out: Optional[PrefillOutput] = None) -> PrefillOutput:
    """Logical mask skipping over every causal block (``cosa_block_mask_prefill``);
    block_mask is int32 [B][Hq][NQB][words] holding uint32 bit patterns."""
    lib = _lib.load()
    problem._check_qkv(q, k_pool, v_pool)
    dev = problem.device
    rows = (problem.batch, problem.num_q_heads, problem.num_q_tiles())
    _need(block_mask, "block_mask", torch.int32, dev, ndim=4)
    if tuple(block_mask.shape[:3]) != rows:
        raise ValueError(f"block_mask rows {tuple(block_mask.shape[:3])} != {rows}")
    if out is None:
        out = PrefillOutput(
            out=torch.empty_like(q),
            lse=torch.empty((problem.num_q_heads, problem.total_q), dtype=torch.float32,
                            device=dev) if lse else None)
    st = lib.cosa_block_mask_prefill(problem.ref(), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(block_mask), block_mask.shape[-1], _ptr(out.out),
                                     _ptr(out.lse), _stream(dev))
    _lib.check(st, "cosa_block_mask_prefill")
    return out
