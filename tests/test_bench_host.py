"""Host-side recounts that bench.py's roofline rests on (no GPU): the latent
nearest-neighbour roots that order the grouped attention's queries, and the
union sizes of the groups, each against a brute-force statement on small
inputs."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _roots_brute(x: np.ndarray) -> np.ndarray:
    """Nearest other query by squared distance (lowest index on ties), then
    follow the chain until it reaches a mutual pair; the pair's lower index."""
    n = x.shape[0]
    xi = x.astype(np.int64)
    nn = np.arange(n)
    for i in range(n):
        best, bj = None, i
        for j in range(n):
            if j == i:
                continue
            d = int(((xi[i] - xi[j]) ** 2).sum())
            if best is None or d < best:
                best, bj = d, j
        nn[i] = bj
    roots = np.empty(n, dtype=np.int64)
    for i in range(n):
        seen, a = set(), i
        while a not in seen:
            seen.add(a)
            a = nn[a]
        # a is on the cycle the chain ends in: a mutual pair (or a lone query)
        roots[i] = min(a, nn[a])
    return roots


@pytest.mark.parametrize("seed,n,spread", [(1, 40, 127), (2, 33, 3), (3, 2, 50), (4, 1, 9), (5, 64, 1)])
def test_latent_nn_roots_match_brute_force(seed, n, spread):
    rng = np.random.default_rng(seed)
    x = rng.integers(-spread, spread + 1, size=(n, 64)).astype(np.int8)
    if n >= 8:
        x[n // 2] = x[0]          # exact duplicates: distance 0, ties to the lowest index
        x[n // 2 + 1] = x[0]
    assert np.array_equal(bench.latent_nn_roots(x), _roots_brute(x))


def test_latent_nn_roots_all_equal():
    """Every query has every other at distance 0: each one's neighbour is the
    lowest other index, so queries 0 and 1 are the mutual pair of everyone."""
    x = np.full((9, 64), 5, dtype=np.int8)
    assert np.array_equal(bench.latent_nn_roots(x), np.zeros(9, dtype=np.int64))


def test_grouped_unions_by_rows():
    """Union sizes of the row order (first long-range key, MinHash, index) on
    hand-made rows: each group's union is the distinct long-range keys of its
    four queries, whatever order they are taken in."""
    wl = bench.S.WORKLOADS["tiny_flat"]          # G = 4: groups of four queries
    t0, n = 100000, 12
    rng = np.random.default_rng(7)
    max_sel = wl.budget + wl.window + wl.sinks
    idx = np.full((n, max_sel), -1, dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    rows = []
    for q in range(n):
        t = t0 + q
        lr = np.sort(rng.choice(50000, size=int(rng.integers(0, 40)), replace=False)).astype(np.int32)
        ws = t - wl.window + 1
        fixed = np.concatenate([np.arange(wl.sinks), np.arange(ws, t + 1)]).astype(np.int32)
        row = np.concatenate([lr, fixed])
        idx[q, :row.size] = row
        cnt[q] = row.size
        rows.append(set(lr.tolist()))
    unions, lr_cnt = bench.grouped_unions(wl, t0, idx, cnt)
    assert lr_cnt.tolist() == [len(r) for r in rows]
    # the groups partition the queries; their union sizes sum to at least the
    # distinct keys overall and at most the entries
    assert len(unions) == n // 4
    assert int(unions.sum()) <= int(lr_cnt.sum())
    assert int(unions.sum()) >= len(set().union(*rows))
    # brute force over the order the function states
    first = np.where(lr_cnt > 0, idx[:, 0].astype(np.int64), (1 << 28) - 1)
    mh = np.array([int(bench._grp_mix(idx[q, :lr_cnt[q]].astype(np.uint64) >> np.uint64(2)).min()) >> 16
                   if lr_cnt[q] > 0 else 0xFFFF for q in range(n)], dtype=np.int64)
    order = sorted(range(n), key=lambda q: (first[q], mh[q], q))
    want = [len(set().union(*(rows[q] for q in order[g:g + 4]))) for g in range(0, n, 4)]
    assert unions.tolist() == want
