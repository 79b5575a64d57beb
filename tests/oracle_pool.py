"""Worker processes for the oracle side of the full-size parity tests.

The oracle's translated retrieval is a Python loop of small fp64 products, so
the tests spread it over processes: each worker regenerates the seeded
workload itself (the same generator the tests use), compresses the block-rows
it is given with the oracle and applies them for the given targets.  Workers
come from a forkserver, fresh processes that never touch the GPU; they import
only numpy, the oracle and the workload generator.

Rows whose kept set legitimately differs from the oracle's at an ambiguous cut
are evaluated with the GPU's own kept set and kept mass (`overrides`), so every
compared row goes through the oracle's retrieval step.
"""
from __future__ import annotations

import dataclasses
import multiprocessing as mp
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from threadpoolctl import threadpool_limits

from oracle import mapflow_oracle as orc
from cross_model_sparse_amd import workloads as wlmod

_cache: Dict[Tuple, "wlmod.Workload"] = {}


def workers() -> int:
    """Oracle processes to use: the machine's CPU share (16 for one GPU), at most 8."""
    return max(1, min(8, (os.cpu_count() or 2) // 2))


def regraded(rr: "orc.RowResult", kept: Sequence[int], kmass: np.ndarray) -> "orc.RowResult":
    """The oracle row with the GPU's kept set and kept mass in place of its own."""
    sel = dataclasses.replace(rr.sel, kept=sorted(int(J) for J in kept))
    return dataclasses.replace(rr, sel=sel, kmass=np.asarray(kmass, dtype=np.float64))


def _workload(key: Tuple) -> "wlmod.Workload":
    if key not in _cache:
        _cache.clear()
        kind, idx = key
        _cache[key] = wlmod.make_config(idx)
    return _cache[key]


def _apply_task(args):
    # one BLAS thread per worker: the products are small, and several workers
    # with a full thread pool each would oversubscribe the cores
    with threadpool_limits(1):
        return _apply_rows(*args)


def _apply_rows(key, rows, targets, overrides, renorm, codec):
    wl = _workload(key)
    B = wl.spec.B
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, wl.spec.p, wl.bias(), rows=rows)
    for k, (kept, km) in overrides.items():
        if k in res:
            res[k] = regraded(res[k], kept, km)
    return orc.apply(res, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv, renorm=renorm,
                     targets=targets, rows=rows, codec=codec)


def apply_config(idx: int, rows: Sequence[Tuple[int, int]], targets: Sequence[int],
                 overrides: Optional[Dict[Tuple[int, int, int], Tuple[List[int], np.ndarray]]] = None,
                 renorm: bool = True, codec: Optional[str] = None,
                 progress=None) -> Dict[Tuple[int, int, int], np.ndarray]:
    """Oracle outputs {(t, s, I): [rows, d]} of workload `idx` for the given
    block-rows and targets, computed in worker processes."""
    overrides = overrides or {}
    n = workers()
    chunks = [list(rows[i::n]) for i in range(n) if rows[i::n]]
    ctx = mp.get_context("forkserver")
    tasks = [(("config", idx), c, list(targets),
              {k: v for k, v in overrides.items() if (k[1], k[2]) in set(c)}, renorm, codec)
             for c in chunks]
    out: Dict[Tuple[int, int, int], np.ndarray] = {}
    with ctx.Pool(len(chunks)) as pool:
        # bounded wait: a worker that cannot start would otherwise be respawned forever
        for i, r in enumerate([pool.apply_async(_apply_task, (t,)) for t in tasks]):
            out.update(r.get(timeout=900))
            if progress:
                progress(f"  oracle retrieval: {i + 1} of {len(tasks)} worker shares done")
    return out
