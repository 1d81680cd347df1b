"""CPU fp64 oracle for CoSA block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
header, table or constant with the HIP library; the only thing both sides see
is the seeded input generator in ``cosa_inputs`` (random draws and layout, no
method arithmetic).

Sources.  The method is described by the CoSA paper ("CoSA: Accelerating
Long-Context Inference via Proxy-Kernel Co-Designed Sparse Attention"), whose
text is available on the paperpeel.com page (sections §3-§4, App. C-D) and
summarised on the researchpod.app page.  The pages give the method in prose;
equations (1)-(5), the body of §4.2 and Algorithm A are not in the text.  Where
the text is silent the oracle takes the plainest reading, listed per function.

Modules
-------
``paging``  de-page a paged KV pool into per-sequence key/value arrays.
``dense``   dense causal softmax attention (textbook definition).
``kap``     Kernel-Aware Proxy: pooled scores, HRM flags, flag-grouped
            ordering and the stage-1 budget truncation.
``osk``     Ordered-Skipping Kernel: sequential online-softmax loop over the
            ordered mask with the tile-wide in-kernel skip, and an independent
            closed form of the same result.
``fidelity`` the KAP kept set against the top-k blocks by exact attention
            mass at a matched budget (IoU, mass recall).

Pinning.  Each function is pinned by ``tests/test_oracle_*.py`` (``-m "not gpu"``)
to closed forms, library routines (``torch`` SDPA in float64 on the CPU),
brute force on tiny inputs, invariants the pages state, and hand-derived
golden cases under ``tests/golden/``.  "Parity unpinned": the exact formula
of the paper's block ranking score and of its Eq. (5) threshold are not
printed on the pages; the oracle is pinned to the readings it states, not to
the paper's own numbers (none are printed).

All floating point here is float64.  Inputs are the bf16-rounded values the
GPU sees, widened exactly to float64.
"""
from . import dense, fidelity, kap, osk, paging  # noqa: F401
