"""Pins for the CPU oracle: it is checked against things other than itself.

Each test ties one oracle function to an independent fact: exact rational
rounding, hand-worked fixtures under tests/golden/, brute-force enumeration
in plain Python, closed forms, and special cases that reduce to a library
routine.  All CPU only.
"""
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- rounding
def test_rhe_div_exhaustive_against_fraction():
    S = np.arange(-600, 601, dtype=np.int64)
    for n in range(1, 70):
        got = O.rhe_div(S, n)
        want = np.array([round(Fraction(int(s), n)) for s in S])   # Python rounds halves to even
        assert np.array_equal(got, want), n


def test_pool_against_fraction_means():
    rng = np.random.default_rng(1)
    for p in (1, 2, 3, 4, 5, 8):
        x = rng.integers(-128, 128, size=(p * 37 + (p - 1), 6))
        got = O.pool(x, p)
        assert got.shape == (37, 6)
        for g in range(37):
            for d in range(6):
                s = int(x[g * p:(g + 1) * p, d].sum())
                assert got[g, d] == round(Fraction(s, p))


# ------------------------------------------------------------------ k-means
def _brute_assign(X, mu):
    """Plain-Python nearest centroid, lowest index on ties."""
    out = []
    for x in X.tolist():
        best, bi = None, -1
        for c, m in enumerate(mu.tolist()):
            d = sum((a - b) * (a - b) for a, b in zip(x, m))
            if best is None or d < best:
                best, bi = d, c
        out.append(bi)
    return np.array(out)


def _frac_mean(rows):
    n = len(rows)
    return [round(Fraction(int(sum(r[d] for r in rows)), n)) for d in range(len(rows[0]))]


def test_kmeans_golden_tie():
    g = _golden("hand_kmeans_tie.json")
    mu, a = O.kmeans(np.array(g["X"]), g["C"], g["iters"])
    assert a.tolist() == g["assign"]
    assert mu.tolist() == g["centroids"]


def test_kmeans_single_cluster_is_rounded_mean():
    rng = np.random.default_rng(2)
    X = rng.integers(-128, 128, size=(50, 8))
    mu, a = O.kmeans(X, 1, 3)
    assert (a == 0).all()
    assert mu[0].tolist() == _frac_mean(X.tolist())


def test_kmeans_one_cluster_per_vector_is_identity():
    rng = np.random.default_rng(3)
    X = rng.integers(-128, 128, size=(32, 8))
    assert len({tuple(r) for r in X.tolist()}) == 32
    mu, a = O.kmeans(X, 32, 4)
    assert a.tolist() == list(range(32))
    assert np.array_equal(mu, X)


@pytest.mark.parametrize("iters", [1, 2, 3])
def test_kmeans_steps_against_brute_force(iters):
    rng = np.random.default_rng(10 + iters)
    # coarse values make exact distance ties frequent
    X = rng.integers(-3, 4, size=(48, 3)) * 2
    C = 6
    mu_prev, _ = O.kmeans(X, C, iters - 1) if iters > 1 else (X[np.arange(C) * (48 // C)], None)
    mu, a = O.kmeans(X, C, iters)
    assert a.tolist() == _brute_assign(X, mu_prev).tolist()
    for c in range(C):
        rows = X[a == c].tolist()
        want = _frac_mean(rows) if rows else mu_prev[c].tolist()
        assert mu[c].tolist() == want, c


# ---------------------------------------------------------------- index
def test_index_golden():
    g = _golden("hand_index_select.json")
    pr = g["params"]
    latk = np.array(g["latk"])
    idx = O.build_index(latk, len(latk), O.IndexParams(pr["pool"], pr["block"], pr["buckets"],
                                                       pr["iters"]))
    assert idx.pooled.tolist() == g["index"]["pooled"]
    assert idx.centroids.tolist() == g["index"]["centroids"]
    assert [m.tolist() for m in idx.members] == g["index"]["members"]


def test_select_golden():
    g = _golden("hand_index_select.json")
    pr = g["params"]
    latk = np.array(g["latk"])
    idx = O.build_index(latk, len(latk), O.IndexParams(pr["pool"], pr["block"], pr["buckets"],
                                                       pr["iters"]))
    sp = O.SelectParams(**g["select_params"])
    for case in g["queries"]:
        got = O.select(idx, np.array(case["q"]), case["t"], sp)
        assert got.tolist() == case["sel"], case["why"]


def _random_index(seed, T, p, N, C, iters, dim=4, lo=-6, hi=7, tree=None):
    rng = np.random.default_rng(seed)
    latk = rng.integers(lo, hi, size=(T, dim))
    params = O.IndexParams(p, N, C, iters, *(tree or (0, 0, 0)))
    return latk, O.build_index(latk, T, params)


def _brute_select(idx, latk, q, t, sp):
    """Enumerate every (bucket, key) pair, order by (score desc, bucket asc,
    key asc), keep the first `budget` eligible keys; add window and sinks."""
    p = idx.params.pool
    pairs = []
    cands = O.candidates(idx, q, sp, t)
    for beta in cands.tolist():
        s = sum(int(a) * int(b) for a, b in zip(q, idx.centroids[beta]))
        for g in idx.members[beta].tolist():
            for r in range(p):
                j = g * p + r
                if sp.sinks <= j <= t - sp.window:
                    pairs.append((-s, beta, j))
    pairs.sort()
    sel = {j for _, _, j in pairs[: sp.budget]}
    sel |= set(range(max(0, t - sp.window + 1), t + 1))
    sel |= set(range(0, min(sp.sinks, t + 1)))
    return sorted(sel)


@pytest.mark.parametrize("seed", range(6))
def test_select_against_enumeration(seed):
    T = 64 + seed * 7
    latk, idx = _random_index(seed, T, p=2, N=8, C=3, iters=2)
    rng = np.random.default_rng(100 + seed)
    for _ in range(12):
        sp = O.SelectParams(budget=int(rng.integers(1, 20)), window=int(rng.integers(2, 9)),
                            sinks=int(rng.integers(0, 5)))
        t = int(rng.integers(0, T))
        q = rng.integers(-5, 6, size=latk.shape[1])
        assert O.select(idx, q, t, sp).tolist() == _brute_select(idx, latk, q, t, sp)


@pytest.mark.parametrize("seed", range(3))
def test_position_dependent_budget_against_enumeration(seed):
    """Before early_until the query keeps early_budget long-range keys, from
    there on budget: each side against the plain enumeration with that budget."""
    T = 72 + seed * 5
    latk, idx = _random_index(20 + seed, T, p=2, N=8, C=3, iters=2)
    rng = np.random.default_rng(200 + seed)
    switch = T // 2
    sp = O.SelectParams(budget=14, window=4, sinks=2, early_budget=5, early_until=switch)
    for t in [0, 3, switch - 2, switch - 1, switch, switch + 1, T - 1]:
        q = rng.integers(-5, 6, size=latk.shape[1])
        b = 5 if t < switch else 14
        assert O.select(idx, q, t, sp).tolist() == \
            _brute_select(idx, latk, q, t, O.SelectParams(budget=b, window=4, sinks=2))


def test_select_count_window_sinks_causal_nesting():
    T = 16384
    latk, idx = _random_index(7, T, p=4, N=256, C=16, iters=3, dim=8, lo=-20, hi=21)
    sp = O.SelectParams(budget=300, window=64, sinks=4)
    rng = np.random.default_rng(8)
    for t in [0, 1, 3, 4, 63, 64, 67, 68, 69, 200, 371, 372, 373, 1000, T - 1] + \
            rng.integers(0, T, 10).tolist():
        q = rng.integers(-30, 31, size=8)
        sel = O.select(idx, q, t, sp)
        assert len(sel) == min(t + 1, sp.budget + sp.window + sp.sinks)
        assert sel.max() <= t and len(np.unique(sel)) == len(sel)
        assert set(range(max(0, t - sp.window + 1), t + 1)) <= set(sel.tolist())
        assert set(range(min(sp.sinks, t + 1))) <= set(sel.tolist())
        bigger = O.select(idx, q, t, O.SelectParams(budget=500, window=64, sinks=4))
        assert set(sel.tolist()) <= set(bigger.tolist())


def test_singleton_buckets_equal_exact_topk():
    """p = 1 and one bucket per vector: selection = exact top-k of per-key scores."""
    T, N = 512, 64
    rng = np.random.default_rng(9)
    latk = rng.integers(-100, 101, size=(T, 8))
    for b in range(T // N):
        assert len({tuple(r) for r in latk[b * N:(b + 1) * N].tolist()}) == N
    idx = O.build_index(latk, T, O.IndexParams(1, N, N, 2))
    # the second setting keeps 9 long-range keys for queries before position 251
    for sp, early in ((O.SelectParams(budget=37, window=16, sinks=3), {}),
                      (O.SelectParams(37, 16, 3, 0, 9, 251), {100: 9, 250: 9})):
        for t in [100, 250, 511]:
            q = rng.integers(-100, 101, size=8)
            keys = np.arange(sp.sinks, t - sp.window + 1)
            sc = latk[keys] @ q
            top = keys[np.lexsort((keys, -sc))][: early.get(t, 37)]
            want = set(top.tolist()) | set(range(t - sp.window + 1, t + 1)) | set(range(sp.sinks))
            assert O.select(idx, q, t, sp).tolist() == sorted(want)
            assert O.dense_select(latk, q, t, sp).tolist() == sorted(want)


def test_tree_with_full_branching_equals_flat():
    T = 4 * 16 * 6 + 50            # 6 full blocks of 16 pooled vectors + a tail; groups of 2 blocks
    latk = np.random.default_rng(11).integers(-30, 31, size=(T, 6))
    flat = O.build_index(latk, T, O.IndexParams(4, 16, 4, 2))
    tree = O.build_index(latk, T, O.IndexParams(4, 16, 4, 2, 2, 3, 2))
    assert tree.n_grp == 3 and tree.sup_centroids.shape[0] == 9
    assert np.array_equal(flat.centroids, tree.centroids)
    rng = np.random.default_rng(12)
    for _ in range(10):
        t = int(rng.integers(0, T))
        q = rng.integers(-30, 31, size=6)
        sp_f = O.SelectParams(budget=40, window=8, sinks=2)
        sp_t = O.SelectParams(budget=40, window=8, sinks=2, tree_top=9)
        assert np.array_equal(O.select(flat, q, t, sp_f), O.select(tree, q, t, sp_t))


def _brute_tree_walk(tree, q, t, sp):
    """Plain-Python Tree walk: nodes ranked by (score desc, id asc) with
    scores summed term by term; a level takes its quota of nodes, then more
    while the keys under the nodes taken (plus every key under no node of
    that level) that satisfy sinks <= j <= t - window, counted one key id at
    a time, stay below the budget.  Returns (candidate leaves, supers taken,
    top nodes taken)."""
    p = tree.params.pool
    B = sp.budget_at(t)

    def dot(a, b):
        return sum(int(x) * int(y) for x, y in zip(a, b))

    def n_elig(leaves):
        return sum(1 for lf in leaves for g in tree.members[lf].tolist() for r in range(p)
                   if sp.sinks <= g * p + r <= t - sp.window)

    def leaves_of(sups):
        return [lf for s in sups for lf in tree.sup_members[s].tolist()]

    loose = list(range(tree.covered_leaves(), tree.n_bkt))
    sups = list(range(len(tree.sup_centroids)))
    tops = []
    if tree.params.tree2_group > 0:
        loose_sup = list(range(tree.covered_supers(), len(tree.sup_centroids)))
        held = n_elig(loose) + n_elig(leaves_of(loose_sup))
        for n in sorted(range(len(tree.top_centroids)), key=lambda n: (-dot(q, tree.top_centroids[n]), n)):
            if len(tops) >= sp.tree2_top and held >= B:
                break
            tops.append(n)
            held += n_elig(leaves_of(tree.top_members[n].tolist()))
        sups = sorted({s for n in tops for s in tree.top_members[n].tolist()} | set(loose_sup))
    held = n_elig(loose)
    taken = []
    for s in sorted(sups, key=lambda s: (-dot(q, tree.sup_centroids[s]), s)):
        if len(taken) >= sp.tree_top and held >= B:
            break
        taken.append(s)
        held += n_elig(tree.sup_members[s].tolist())
    return sorted(set(loose) | set(leaves_of(taken))), taken, tops


@pytest.mark.parametrize("nblk", [6, 7])
def test_tree_candidates_against_brute_force(nblk):
    """The walk against plain-Python enumeration, with budgets the best
    tree_top supers already hold (no fill) and budgets they do not (the walk
    continues in score order); both cases occur.  With 7 blocks the last one
    is outside the complete groups: its leaves are candidates whose keys
    count towards the budget from the start."""
    T = 4 * 16 * nblk + 50
    latk = np.random.default_rng(13).integers(-30, 31, size=(T, 6))
    tree = O.build_index(latk, T, O.IndexParams(4, 16, 4, 2, 2, 3, 2))
    # every leaf of a complete group is in exactly one super cluster
    cov = np.sort(np.concatenate(tree.sup_members))
    assert cov.tolist() == list(range(tree.covered_leaves()))
    rng = np.random.default_rng(14)
    filled = quota = 0
    for R in (1, 2, 4):
        for B in (8, 60, 200, 2000):
            q = rng.integers(-30, 31, size=6)
            t = T - 1 - int(rng.integers(0, 200))
            sp = O.SelectParams(budget=B, window=8, sinks=2, tree_top=R)
            want, taken, _ = _brute_tree_walk(tree, q, t, sp)
            assert O.candidates(tree, q, sp, t).tolist() == want
            # the same query with the budget equal to what the loose leaves and
            # the best R + 1 supers hold: the walk stops right there
            order = sorted(range(len(tree.sup_centroids)),
                           key=lambda s: (-int(np.dot(q, tree.sup_centroids[s])), s))
            leaves = list(range(tree.covered_leaves(), tree.n_bkt)) + \
                [lf for s in order[:R + 1] for lf in tree.sup_members[s].tolist()]
            exact = sum(len(O.eligible_keys(O.bucket_keys(tree, lf), t, sp)) for lf in leaves)
            spx = O.SelectParams(budget=exact, window=8, sinks=2, tree_top=R)
            want_x, taken_x, _ = _brute_tree_walk(tree, q, t, spx)
            assert taken_x == order[:R + 1]
            assert O.candidates(tree, q, spx, t).tolist() == want_x
            assert O.candidates(tree, q, sp, t).tolist() == want
            filled += len(taken) > R
            quota += len(taken) == R
            assert O.select(tree, q, t, sp).tolist() == _brute_select(tree, latk, q, t, sp)
    assert filled and quota


def test_tree_fill_count_and_minimal_walk():
    """With the fill, a Tree selection holds exactly min(t + 1, B + w + s)
    keys, as Flat does; the supers taken are a prefix of the score order,
    and when the walk took more than tree_top of them, the last one was
    needed to reach the budget."""
    T = 4 * 16 * 6 + 50
    latk = np.random.default_rng(15).integers(-30, 31, size=(T, 6))
    tree = O.build_index(latk, T, O.IndexParams(4, 16, 4, 2, 2, 3, 2))
    rng = np.random.default_rng(16)
    p = tree.params.pool
    for t in [0, 5, 9, 10, 40, 100, 250, 384, 385, T - 1] + rng.integers(0, T, 8).tolist():
        for R, B in ((1, 30), (2, 120), (1, 400)):
            q = rng.integers(-30, 31, size=6)
            sp = O.SelectParams(budget=B, window=8, sinks=2, tree_top=R)
            sel = O.select(tree, q, t, sp)
            assert len(sel) == min(t + 1, B + 8 + 2), (t, R, B)
            _, taken, _ = _brute_tree_walk(tree, q, t, sp)
            order = sorted(range(9), key=lambda s: (-int(np.dot(q, tree.sup_centroids[s])), s))
            assert taken == order[:len(taken)]
            if len(taken) > R:
                leaves = list(range(tree.covered_leaves(), tree.n_bkt)) + \
                    [lf for s in taken[:-1] for lf in tree.sup_members[s].tolist()]
                short = sum(len(O.eligible_keys(O.bucket_keys(tree, lf), t, sp)) for lf in leaves)
                assert short < B


def _tree3(seed):
    # 10 full blocks of 16 pooled vectors + a tail; groups of 2 blocks (3 supers
    # each), top groups of 2 groups (2 top nodes each): 2 complete top groups,
    # group 4 outside them
    T = 4 * 16 * 10 + 37
    latk = np.random.default_rng(seed).integers(-30, 31, size=(T, 6))
    prm = O.IndexParams(4, 16, 4, 2, 2, 3, 2, 2, 2, 3)
    return T, latk, O.build_index(latk, T, prm)


def test_tree3_top_level_partitions_and_means():
    T, latk, tree = _tree3(21)
    assert tree.n_grp == 5 and tree.n_grp2 == 2 and tree.top_centroids.shape[0] == 4
    assert tree.covered_supers() == 12
    cov = np.sort(np.concatenate(tree.top_members))
    assert cov.tolist() == list(range(12))
    # after the last update every non-empty node's centroid is the rounded
    # (half-even) mean of the super centroids assigned to it
    for n, m in enumerate(tree.top_members):
        if len(m):
            assert tree.top_centroids[n].tolist() == _frac_mean(tree.sup_centroids[m].tolist())


def test_tree3_full_top_branching_equals_two_levels():
    T, latk, tree3 = _tree3(22)
    tree2 = O.build_index(latk, T, O.IndexParams(4, 16, 4, 2, 2, 3, 2))
    assert np.array_equal(tree2.sup_centroids, tree3.sup_centroids)
    rng = np.random.default_rng(23)
    for R in (1, 3, 7):
        for _ in range(4):
            q = rng.integers(-30, 31, size=6)
            t = int(rng.integers(0, T))
            sp2 = O.SelectParams(budget=40, window=8, sinks=2, tree_top=R)
            sp3 = O.SelectParams(budget=40, window=8, sinks=2, tree_top=R, tree2_top=4)
            assert np.array_equal(O.select(tree2, q, t, sp2), O.select(tree3, q, t, sp3))


def test_tree3_candidates_against_brute_force():
    T, latk, tree = _tree3(24)
    rng = np.random.default_rng(25)
    filled_top = 0
    for R2, R in ((1, 1), (1, 3), (2, 2), (3, 5)):
        for B in (10, 150, 1200):
            q = rng.integers(-30, 31, size=6)
            t = T - 1 - int(rng.integers(0, 100))
            sp = O.SelectParams(budget=B, window=8, sinks=2, tree_top=R, tree2_top=R2)
            want, _, tops = _brute_tree_walk(tree, q, t, sp)
            filled_top += len(tops) > R2
            assert O.candidates(tree, q, sp, t).tolist() == want
            assert O.select(tree, q, t, sp).tolist() == _brute_select(tree, latk, q, t, sp)
            assert len(O.select(tree, q, t, sp)) == min(t + 1, B + 8 + 2)
    assert filled_top


def _brute_lloyd(X, C, iters):
    """Plain-Python Lloyd k-means: centroid c starts at vector c * (N // C);
    each iteration assigns by brute force (lowest index on ties), then sets
    every non-empty centroid to the exact rational mean of its members,
    rounded half to even; an empty centroid is kept."""
    rows = [[int(v) for v in r] for r in np.asarray(X).tolist()]
    stride = len(rows) // C
    mu = [rows[c * stride][:] for c in range(C)]
    a = []
    for _ in range(iters):
        a = _brute_assign(np.array(rows), np.array(mu)).tolist()
        for c in range(C):
            mine = [r for r, ac in zip(rows, a) if ac == c]
            if mine:
                mu[c] = _frac_mean(mine)
    return mu, a


def test_tree_levels_use_their_own_iteration_counts():
    """Leaf, super and top levels run 3, 1 and 2 Lloyd iterations: each upper
    level equals a plain-Python Lloyd over the level below with its own count
    (super members are leaf ids, top members super ids), and the other counts
    give a different result on this input, so swapping them cannot pass."""
    # 29 blocks of 16 pooled vectors (8 buckets each), groups of 4 blocks
    # (6 supers), top groups of 3 groups (4 top nodes): 7 groups, 2 top groups
    T = 4 * 16 * 29 + 37
    latk = np.random.default_rng(32).integers(-40, 41, size=(T, 6))
    prm = O.IndexParams(4, 16, 8, 3, 4, 6, 1, 3, 4, 2)
    idx = O.build_index(latk, T, prm)
    assert idx.n_full == 29 and idx.n_grp == 7 and idx.n_grp2 == 2
    # leaf level: every block with its own count (3)
    for b in range(idx.n_full):
        mu, a = _brute_lloyd(idx.pooled[b * 16:(b + 1) * 16], 8, 3)
        assert idx.centroids[b * 8:(b + 1) * 8].tolist() == mu
    levels = (
        ("super", idx.centroids, 4 * 8, 6, idx.n_grp, 1, idx.sup_centroids, idx.sup_members),
        ("top", idx.sup_centroids, 3 * 6, 4, idx.n_grp2, 2, idx.top_centroids, idx.top_members),
    )
    for name, below, per_grp, S, n_grp, own, cent, members in levels:
        differs = {k: False for k in (1, 2, 3) if k != own}
        for g in range(n_grp):
            X = below[g * per_grp:(g + 1) * per_grp]
            mu, a = _brute_lloyd(X, S, own)
            assert cent[g * S:(g + 1) * S].tolist() == mu, (name, g)
            for c in range(S):
                want = [g * per_grp + i for i, ac in enumerate(a) if ac == c]
                assert members[g * S + c].tolist() == want, (name, g, c)
            for k in differs:
                mk, ak = _brute_lloyd(X, S, k)
                differs[k] |= (mk != mu) or (ak != a)
        assert all(differs.values()), (name, differs)


def test_index_is_prefix_function():
    """The index over keys [0, T') depends only on those keys (cache-consistent)."""
    latk = np.random.default_rng(15).integers(-40, 41, size=(3000, 4))
    params = O.IndexParams(4, 64, 8, 3)
    cache = {}
    for Tp in (0, 5, 255, 256, 257, 1024, 2999):
        a = O.build_index(latk, Tp, params, cache)
        b = O.build_index(latk[:Tp].copy(), Tp, params)
        assert np.array_equal(a.centroids, b.centroids)
        assert [m.tolist() for m in a.members] == [m.tolist() for m in b.members]
        # every complete pooled group is in exactly one bucket
        allm = np.sort(np.concatenate(a.members)) if a.members else np.zeros(0)
        assert allm.tolist() == list(range(Tp // 4))


# ---------------------------------------------------------------- attention
def test_attention_golden():
    g = _golden("hand_attention.json")
    out = O.attend(np.array([g["q"]]), np.array(g["K"])[:, None, :], np.array(g["V"])[:, None, :], 1)
    assert np.allclose(out[0], g["out"], rtol=0, atol=1e-12)


def test_attention_full_selection_is_causal_sdpa():
    """Selecting every key 0..t reduces to textbook causal attention."""
    rng = np.random.default_rng(16)
    T, Hq, Hkv, D = 40, 6, 2, 16
    q = rng.standard_normal((T, Hq, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2),
        torch.from_numpy(np.repeat(K, Hq // Hkv, axis=1)).permute(1, 0, 2),
        torch.from_numpy(np.repeat(V, Hq // Hkv, axis=1)).permute(1, 0, 2),
        is_causal=True).permute(1, 0, 2).numpy()
    for t in range(T):
        sel = np.arange(t + 1)
        got = O.attend(q[t], K[sel], V[sel], Hkv)
        assert np.allclose(got, ref[t], rtol=1e-12, atol=1e-12)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((8, 32))
    K = rng.standard_normal((1, 4, 32))
    V = rng.standard_normal((1, 4, 32))
    out = O.attend(q, K, V, 4)
    for h in range(8):
        assert np.array_equal(out[h], V[0, h // 2])


def test_bf16_decode_exact():
    vals = np.array([1.0, -2.5, 0.0078125, 3.140625, -0.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(bits), vals.astype(np.float64))
    t = torch.tensor(vals).to(torch.bfloat16)
    assert np.array_equal(O.bf16_to_f64(t.view(torch.int16).numpy()), t.double().numpy())
