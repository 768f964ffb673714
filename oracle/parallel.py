"""Run the fp64 oracle over many (batch, head) units at once.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite and
the benchmark's CPU-baseline leg use it; the product never does.

The oracle evaluates one (batch, head) unit at a time with numpy; its matrix
products and element-wise passes release the interpreter lock, so a pool of
threads, each with single-threaded BLAS, evaluates independent units on as
many host cores.  Nothing here changes what the oracle computes: each unit is
the oracle's own attention_rows over all query rows of that unit.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .bigbird_oracle import (attention_backward_unit, attention_rows, block_adjacency, check_rand_idx,
                             num_blocks)

# At most 16 worker threads: a host shared between GPUs gives each GPU's
# process about that many cores, whatever the machine-wide count says.
MAX_WORKERS = 16


def host_workers() -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def forward_units(q, k, v, pad, rand_idx, block: int, units=None, workers: int = 0,
                  out=None, rows_per_group: int = 0, query_mask: bool = False):
    """Oracle output of `units` ((b, h) pairs; default all) into `out`
    (float64 [B, H, L, d], allocated as NaN when None).  q, k, v: arrays
    [B, H, L, d] (any real dtype, upcast per unit); pad: [B, L] or None."""
    from threadpoolctl import threadpool_limits
    B, H, L, d = q.shape
    nb = num_blocks(L, block)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    if out is None:
        out = np.full((B, H, L, d), np.nan)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    adj = {h: block_adjacency(rand_idx[h], nb) for h in {h for _, h in units}}
    group = rows_per_group or (2048 if L > 8192 else L)

    def one(bh):
        b, h = bh
        qb, kb, vb = (np.asarray(t[b, h], np.float64) for t in (q, k, v))
        pb = None if pad is None else np.asarray(pad[b])
        for r0 in range(0, L, group):
            rows = np.arange(r0, min(L, r0 + group))
            out[b, h, rows] = attention_rows(qb, kb, vb, pb, adj[h], block, rows, query_mask)
        return bh

    n = workers or host_workers()
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=n) as ex:
            for _ in ex.map(one, units):
                pass
    return out


def backward_units(q, k, v, pad, rand_idx, block: int, dout, units=None, workers: int = 0,
                   query_mask: bool = False):
    """Oracle gradients (dq, dk, dv) of `units` ((b, h) pairs; default all), each
    float64 [B, H, L, d] with NaN outside the units; the oracle's own
    attention_backward_unit per unit, units spread over host threads."""
    from threadpoolctl import threadpool_limits
    B, H, L, d = q.shape
    nb = num_blocks(L, block)
    rand_idx = np.asarray(rand_idx)
    r = rand_idx.shape[2] if rand_idx.ndim == 3 else 0
    check_rand_idx(rand_idx, H, L, block, r)
    grads = [np.full((B, H, L, d), np.nan) for _ in range(3)]
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    adj = {h: block_adjacency(rand_idx[h], nb) for h in {h for _, h in units}}
    group = 2048 if L > 8192 else L

    def one(bh):
        b, h = bh
        res = attention_backward_unit(q[b, h], k[b, h], v[b, h], dout[b, h],
                                      None if pad is None else np.asarray(pad[b]), adj[h], block, group,
                                      query_mask)
        for g, x in zip(grads, res):
            g[b, h] = x
        return bh

    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers or host_workers()) as ex:
            for _ in ex.map(one, units):
                pass
    return grads
