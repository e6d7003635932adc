"""Oracle index of a long context, built block by block in worker processes.

TEST INFRASTRUCTURE ONLY (used by full-size parity tests and the benchmark's
CPU-baseline leg).  Full blocks are independent, so each worker regenerates
the latent keys of a range of blocks with the seeded generator, pools them
and runs the oracle's k-means on each block; the parent assembles the
per-block cache that ``oracle.build_index`` consumes.  No arithmetic here
beyond calling the oracle.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np


def _work(args):
    import torch
    torch.set_num_threads(1)
    import lsa_synth as S
    from . import lsa_oracle as O
    wl_name, seq, data_cfg, b_lo, b_hi = args
    wl = S.WORKLOADS[wl_name]
    g = S.Synth(wl, seq=seq, data_cfg=data_cfg)
    kpb = wl.pool * wl.block
    lat = g.latk(b_lo * kpb, b_hi * kpb, chunk=1 << 17).numpy()
    P = O.pool(lat, wl.pool)
    out = []
    for j in range(b_hi - b_lo):
        mu, a = O.kmeans(P[j * wl.block:(j + 1) * wl.block], wl.buckets, wl.iters)
        out.append((b_lo + j, mu, a))
    return b_lo, lat, out


def build_cache_parallel(wl_name: str, T: int, pool, seq: int = 0, data_cfg=None,
                         blocks_per_task: int = 4) -> Tuple[Dict, np.ndarray]:
    """Per-block k-means cache for keys [0, T) and the latent keys themselves.

    ``pool`` is a multiprocessing pool (or None to run in-process).
    """
    import lsa_synth as S
    wl = S.WORKLOADS[wl_name]
    kpb = wl.pool * wl.block
    n_full = (T // wl.pool) // wl.block
    tasks = [(wl_name, seq, data_cfg, b, min(n_full, b + blocks_per_task))
             for b in range(0, n_full, blocks_per_task)]
    results = pool.map(_work, tasks) if pool is not None else [_work(t) for t in tasks]
    results.sort(key=lambda r: r[0])
    cache: Dict = {}
    lats = []
    for _, lat, out in results:
        lats.append(lat)
        for b, mu, a in out:
            cache[("blk", b)] = (mu, a)
    g = S.Synth(wl, seq=seq, data_cfg=data_cfg)
    if T > n_full * kpb:
        lats.append(g.latk(n_full * kpb, T).numpy())
    latk = np.concatenate(lats) if lats else np.zeros((0, wl.dim), np.int8)
    return cache, latk
