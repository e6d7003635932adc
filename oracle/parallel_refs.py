"""Oracle results for many queries at once, computed in worker processes.

TEST INFRASTRUCTURE ONLY (full-size parity tests).  The work is split over a
multiprocessing pool that was forked before anything touched the GPU; each
worker only calls the oracle's own functions (``select``, ``build_index``) on
inputs it receives or regenerates with the seeded generator.
Nothing here does any of the method's arithmetic.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import lsa_oracle as O


def _slim(idx: O.Index) -> O.Index:
    """The index without the arrays selection never reads (pooled vectors and
    the pooled-to-bucket map), to keep what is sent to workers small."""
    dim = idx.pooled.shape[1] if idx.pooled.ndim == 2 else 64
    return dataclasses.replace(idx, pooled=np.zeros((0, dim), np.int64), assign=np.zeros(0, np.int64))


def _select_task(args):
    idx, sp, items = args
    return [O.select(idx, q, t, sp) for q, t in items]


def select_many(pool, idx: O.Index, latq: np.ndarray, positions: Sequence[int],
                sp: O.SelectParams, tasks: int = 16) -> List[np.ndarray]:
    """O.select for query i (latent latq[i], position positions[i]), in order."""
    slim = _slim(idx)
    parts = np.array_split(np.arange(len(positions)), max(1, min(tasks, len(positions))))
    work = [(slim, sp, [(latq[i], int(positions[i])) for i in part]) for part in parts if len(part)]
    res = pool.map(_select_task, work) if pool is not None else [_select_task(w) for w in work]
    return [s for r in res for s in r]


def _decode_task(args):
    """Every step of one decode sequence: the oracle index over the keys up to
    and including the step's new key, and the selection for the new position."""
    import torch
    torch.set_num_threads(1)
    import lsa_synth as S
    wl_name, seq, T0, steps, params, sp, cache = args
    wl = S.WORKLOADS[wl_name]
    g = S.Synth(wl, seq=seq)
    latk = g.latk(0, T0 + steps).numpy()
    lq = g.latq_rows(torch.arange(T0, T0 + steps)).numpy()
    sels = []
    ref, n_pool = None, -1
    for s in range(steps):
        t = T0 + s
        if (t + 1) // params.pool != n_pool:          # the index changes when a pooled group completes
            ref = O.build_index(latk, t + 1, params, cache)
            n_pool = (t + 1) // params.pool
        sels.append(O.select(ref, lq[s], t, sp))
    return sels


def decode_many(pool, wl_name: str, T0: int, steps: int, params: O.IndexParams, sp: O.SelectParams,
                caches: Sequence[Dict]):
    """Per sequence i (one task each): the oracle's selections at positions
    T0 .. T0 + steps - 1, each over the index of the keys up to that position
    (``caches[i]``: the sequence's per-block k-means results, from
    build_cache_parallel)."""
    work = [(wl_name, i, T0, steps, params, sp, caches[i]) for i in range(len(caches))]
    return pool.map(_decode_task, work) if pool is not None else [_decode_task(w) for w in work]
