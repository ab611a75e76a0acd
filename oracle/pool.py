"""Process-pool driver for the fp64 oracle over (batch, head, row-range) units.

Test infrastructure only (see the package doc). It adds no arithmetic: each
unit is ``head_attention_fp64`` on a slice of query rows, the definition
taken from the zyxy.net lecture page (section 1) and the intelliparadigm page
(section 1.1). Work is split over forked worker processes, each limited to
one BLAS thread, so the number of cores used equals the pool size.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import List, Sequence, Tuple

import numpy as np

from .attention import head_attention_fp64, kv_head_of

_SHARED = {}


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _run_unit(unit):
    from threadpoolctl import threadpool_limits

    b, hq, rows = unit
    q, k, v, scale, causal = (_SHARED[x] for x in ("q", "k", "v", "scale", "causal"))
    hk = kv_head_of(hq, q.shape[1], k.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    with threadpool_limits(1):
        O, L = head_attention_fp64(q[b, hq][rows], k[b, hk], v[b, hk], scale, causal, q_pos=rows)
    return b, hq, rows, O, L


def attention_rows_pool(q, k, v, scale: float, causal: bool,
                        units: Sequence[Tuple[int, int, Sequence[int]]], workers: int):
    """Evaluate the oracle on ``units`` = [(b, hq, row_indices), ...] with ``workers`` processes.

    q, k, v are float64 [B,H,N,d] arrays (K/V with Hkv heads). Returns a list
    of (b, hq, rows, O_rows, LSE_rows) in the order of ``units``.
    """
    _SHARED.update(q=q, k=k, v=v, scale=scale, causal=causal)
    try:
        if workers <= 1:
            return [_run_unit(u) for u in units]
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            return pool.map(_run_unit, list(units), chunksize=1)
    finally:
        _SHARED.clear()


def attention_fp64_pool(q, k, v, scale: float, causal: bool, workers: int, rows_per_unit: int = 1024):
    """Full attention (O, LSE) in fp64 using ``workers`` processes."""
    B, Hq, N, _ = q.shape
    units: List[Tuple[int, int, range]] = [
        (b, h, range(r0, min(N, r0 + rows_per_unit)))
        for b in range(B) for h in range(Hq) for r0 in range(0, N, rows_per_unit)
    ]
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty((B, Hq, N), dtype=np.float64)
    for b, h, rows, o, l in attention_rows_pool(q, k, v, scale, causal, units, workers):
        O[b, h, rows] = o
        LSE[b, h, rows] = l
    return O, LSE
