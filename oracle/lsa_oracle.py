"""CPU oracle for the Latent Sparse Attention (LSA) hot path.

TEST INFRASTRUCTURE ONLY.  Plain, slow, step-by-step NumPy code that defines
what the GPU path must compute.  Only the tests, the package's ``smoke()``
entry and the benchmark's CPU-baseline leg may import it; the product path
never does.  It shares no code with the HIP library and never reads anything
the GPU produced.

Sources (cited by page title and passage; the pages are web articles about
the preprint "Latent Sparse Attention: Towards Subquadratic Ultra-Long Context
Attention", arXiv 2610.42147):

* "Latent Sparse Attention: un indice gerarchico per contesti lunghi"
  (mauroscia.it), paragraph on how LSA builds its index: consecutive keys are
  pooled in small groups, the pooled sequence is split into blocks, similar
  vectors in each block are grouped into buckets, each bucket keeps a
  centroid and the indices of its original keys.
* same page, paragraph on the search: the query is compared with the
  centroids to choose the buckets whose keys are fetched; attention then runs
  on the selected keys and values; centroids serve the search only.
* same page, paragraph on the D-LSA configuration: 64-d index
  representations, 4096 long-range keys (outside the recent window) per
  query, plus the 512 most recent keys and 4 sink keys at the start.
* "Prefrontal's Latent Sparse Attention speeds up one attention layer 72x at
  10M tokens" (sysnote.net), section "What it changes": clusters are grouped
  into a hierarchy, a query scores a few clusters per level, walks down the
  tree and only then fetches keys; the attention kernel itself is unchanged.

Where the pages are silent, the readings used here (and listed in the design
notes) are: integer k-means with strided initialisation, squared-L2 assign
with lowest-index ties, round-half-even integer means, empty clusters keep
their centroid; a partial tail block is made of singleton buckets until it
fills; buckets are ranked by (score desc, bucket id asc) and filled key by
key in ascending position up to the budget, the last bucket cut at its
lowest positions; window = the w most recent keys including the query's own
position; causal masking per key; one latent query per token shared by all
its heads; softmax scale 1/sqrt(D); head h reads KV head floor(h*Hkv/Hq).
The Tree walk takes its quota of best nodes per level and keeps taking the
next best while the candidates hold fewer eligible keys than the budget, so
a Tree query fills the same fixed number of keys as a Flat one.

All index arithmetic is exact integer arithmetic (NumPy int64).  Integer dot
products go through float64 matrix products, which are exact here because
every |sum| <= 64 * 128 * 128 < 2**53.  Attention is evaluated in float64 from
the bf16 inputs (which convert to float exactly).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# integer rounding
# --------------------------------------------------------------------------
def rhe_div(s, n):
    """Round-half-even of the exact quotient s/n for integers (n > 0).

    q = floor(s/n), r = s - q*n in [0, n); round up when 2r > n, or when
    2r == n and q is odd.  Works elementwise on int64 arrays.
    """
    s = np.asarray(s, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    q = np.floor_divide(s, n)
    r = s - q * n
    up = (2 * r > n) | ((2 * r == n) & (np.mod(q, 2) == 1))
    return q + up.astype(np.int64)


# --------------------------------------------------------------------------
# index build: pooling, blocks, clustering (mauroscia.it, index paragraph)
# --------------------------------------------------------------------------
def pool(latk: np.ndarray, p: int) -> np.ndarray:
    """Pooled vector g = rounded mean of keys g*p .. g*p+p-1 (int64 [T//p][dim]).

    Keys past the last complete group belong to no pooled vector.
    """
    n = latk.shape[0] // p
    x = np.asarray(latk[: n * p], dtype=np.int64).reshape(n, p, latk.shape[1])
    return rhe_div(x.sum(axis=1), p)


def sq_dist(X: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances [len(X)][len(mu)], exact (int64 result)."""
    Xf = X.astype(np.float64)
    Mf = mu.astype(np.float64)
    d = (Xf * Xf).sum(1)[:, None] - 2.0 * (Xf @ Mf.T) + (Mf * Mf).sum(1)[None, :]
    return d.astype(np.int64)


def kmeans(X: np.ndarray, C: int, iters: int) -> Tuple[np.ndarray, np.ndarray]:
    """Integer Lloyd k-means.  Returns (centroids int64 [C][dim], assign int64 [N]).

    init: centroid c = X[c * (N // C)]; each iteration assigns every vector to
    its nearest centroid (squared L2, lowest index on ties) and then replaces
    each non-empty centroid by the round-half-even mean of its members (an
    empty centroid is kept).  The returned assignment is the last assign step
    and the returned centroids the last update, so every non-empty centroid is
    the rounded mean of its members.
    """
    X = np.asarray(X, dtype=np.int64)
    N = X.shape[0]
    stride = N // C
    mu = X[np.arange(C) * stride].copy()
    assign = np.zeros(N, dtype=np.int64)
    for _ in range(iters):
        assign = np.argmin(sq_dist(X, mu), axis=1)          # first minimum = lowest index
        counts = np.bincount(assign, minlength=C)
        sums = np.zeros_like(mu)
        for d in range(X.shape[1]):
            # per-cluster sums of one coordinate; float64 is exact (|sum| < 2**53)
            sums[:, d] = np.rint(np.bincount(assign, weights=X[:, d].astype(np.float64),
                                             minlength=C)).astype(np.int64)
        ne = counts > 0
        mu[ne] = rhe_div(sums[ne], counts[ne][:, None])
    return mu, assign


@dataclasses.dataclass
class IndexParams:
    pool: int = 4
    block: int = 4096
    buckets: int = 256
    iters: int = 4
    tree_group: int = 0
    tree_super: int = 0
    tree_iters: int = 0
    # third level (sysnote.net "What it changes": clusters are grouped into a
    # hierarchy and a query walks it level by level): the super clusters of
    # each complete run of ``tree2_group`` groups are clustered into
    # ``tree2_super`` top nodes
    tree2_group: int = 0
    tree2_super: int = 0
    tree2_iters: int = 0


@dataclasses.dataclass
class Index:
    """The LSA index over keys [0, T).

    Buckets: full blocks first (block b owns ids b*C .. b*C+C-1), then one
    singleton bucket per pooled vector of the partial tail block.  ``members``
    lists, per bucket, its pooled ids in ascending order; key ids of pooled
    id g are g*p .. g*p+p-1.  Tree: super clusters over the leaf centroids of
    each complete group of ``tree_group`` blocks.
    """
    params: IndexParams
    T: int
    n_pool: int
    n_full: int
    pooled: np.ndarray
    centroids: np.ndarray              # int64 [n_bkt][dim]
    members: List[np.ndarray]          # per bucket: ascending pooled ids
    assign: np.ndarray                 # bucket id of every pooled vector
    n_grp: int = 0
    sup_centroids: Optional[np.ndarray] = None   # int64 [n_sup][dim]
    sup_members: Optional[List[np.ndarray]] = None  # per super: ascending leaf ids
    n_grp2: int = 0
    top_centroids: Optional[np.ndarray] = None   # int64 [n_top][dim] (third level)
    top_members: Optional[List[np.ndarray]] = None  # per top node: ascending super ids

    @property
    def n_bkt(self) -> int:
        return self.centroids.shape[0]

    def covered_leaves(self) -> int:
        """Leaves with id < this value belong to a super cluster."""
        return self.n_grp * self.params.tree_group * self.params.buckets

    def covered_supers(self) -> int:
        """Super clusters with id < this value belong to a top node."""
        return self.n_grp2 * self.params.tree2_group * self.params.tree_super


def build_index(latk: np.ndarray, T: int, params: IndexParams,
                cache: Optional[Dict] = None) -> Index:
    """Index of keys [0, T) of ``latk`` (int8 [>=T][dim]).

    Full blocks are clustered with ``kmeans``; the tail block's pooled
    vectors are singleton buckets.  ``cache`` may hold per-block results
    (full blocks never change once complete), keyed by ('blk', b) and
    ('grp', g).
    """
    p, N, C = params.pool, params.block, params.buckets
    P = pool(latk[:T], p)
    n_pool = P.shape[0]
    n_full = n_pool // N
    cents: List[np.ndarray] = []
    members: List[np.ndarray] = []
    assign = np.zeros(n_pool, dtype=np.int64)
    for b in range(n_full):
        key = ("blk", b)
        if cache is not None and key in cache:
            mu, a = cache[key]
        else:
            mu, a = kmeans(P[b * N:(b + 1) * N], C, params.iters)
            if cache is not None:
                cache[key] = (mu, a)
        cents.append(mu)
        base = b * N
        for c in range(C):
            members.append(base + np.nonzero(a == c)[0].astype(np.int64))
        assign[base:base + N] = b * C + a
    for g in range(n_full * N, n_pool):                      # tail singletons
        cents.append(P[g:g + 1])
        members.append(np.array([g], dtype=np.int64))
        assign[g] = n_full * C + (g - n_full * N)
    dim = latk.shape[1]
    centroids = np.concatenate(cents, axis=0) if cents else np.zeros((0, dim), np.int64)
    idx = Index(params, T, n_pool, n_full, P, centroids, members, assign)
    if params.tree_group > 0:
        G, S = params.tree_group, params.tree_super
        idx.n_grp = n_full // G
        sc, sm = [], []
        for g in range(idx.n_grp):
            key = ("grp", g)
            leaves = centroids[g * G * C:(g + 1) * G * C]
            if cache is not None and key in cache:
                mu, a = cache[key]
            else:
                mu, a = kmeans(leaves, S, params.tree_iters)
                if cache is not None:
                    cache[key] = (mu, a)
            sc.append(mu)
            for c in range(S):
                sm.append(g * G * C + np.nonzero(a == c)[0].astype(np.int64))
        idx.sup_centroids = np.concatenate(sc, axis=0) if sc else np.zeros((0, dim), np.int64)
        idx.sup_members = sm
        if params.tree2_group > 0:
            G2, S2 = params.tree2_group, params.tree2_super
            idx.n_grp2 = idx.n_grp // G2
            tc, tm = [], []
            for g2 in range(idx.n_grp2):
                key = ("grp2", g2)
                sups = idx.sup_centroids[g2 * G2 * S:(g2 + 1) * G2 * S]
                if cache is not None and key in cache:
                    mu, a = cache[key]
                else:
                    mu, a = kmeans(sups, S2, params.tree2_iters)
                    if cache is not None:
                        cache[key] = (mu, a)
                tc.append(mu)
                for c in range(S2):
                    tm.append(g2 * G2 * S + np.nonzero(a == c)[0].astype(np.int64))
            idx.top_centroids = np.concatenate(tc, axis=0) if tc else np.zeros((0, dim), np.int64)
            idx.top_members = tm
    return idx


# --------------------------------------------------------------------------
# selection (mauroscia.it search and budget paragraphs; sysnote.net tree walk)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class SelectParams:
    budget: int = 4096
    window: int = 512
    sinks: int = 4
    tree_top: int = 0
    # position-dependent budget (mauroscia.it D-LSA paragraph: on GLM, Flat
    # takes 2048 long-range keys for queries before position 1M):
    # queries at t < early_until take early_budget long-range keys
    early_budget: int = 0
    early_until: int = 0
    tree2_top: int = 0     # top nodes taken per query (third tree level)

    def budget_at(self, t: int) -> int:
        return self.early_budget if t < self.early_until else self.budget


def bucket_keys(idx: Index, beta: int) -> np.ndarray:
    """Ascending key ids of bucket beta."""
    p = idx.params.pool
    g = idx.members[beta]
    return (g[:, None] * p + np.arange(p)[None, :]).reshape(-1)


def eligible_keys(keys: np.ndarray, t: int, sp: SelectParams) -> np.ndarray:
    """Long-range keys usable by the query at position t: sinks <= j <= t - window."""
    return keys[(keys >= sp.sinks) & (keys <= t - sp.window)]


def scores(cent: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Plain integer dot products q . centroid (int64)."""
    return (cent.astype(np.float64) @ np.asarray(q, dtype=np.float64)).astype(np.int64)


def eligible_count(idx: Index, beta: int, t: int, sp: SelectParams) -> int:
    """Number of long-range keys of bucket beta usable at position t."""
    return int(eligible_keys(bucket_keys(idx, beta), t, sp).size)


def _walk(order: np.ndarray, quota: int, held: int, need: int, weight) -> List[int]:
    """Nodes taken from ``order`` (best first): the first ``quota`` of them,
    then the next ones while the eligible keys held (``held`` to start with,
    plus ``weight(node)`` for every node taken) stay below ``need``."""
    taken: List[int] = []
    for n in order.tolist():
        if len(taken) >= quota and held >= need:
            break
        taken.append(n)
        held += weight(n)
    return taken


def candidates(idx: Index, q: np.ndarray, sp: SelectParams, t: int) -> np.ndarray:
    """Bucket ids the query at position t may draw from: all (Flat) or the
    leaves the Tree walk reaches.

    Tree: super clusters are ranked by (score desc, id asc).  The walk takes
    the ``tree_top`` best, then keeps taking the next best while the
    candidate leaves (the members of the supers taken, plus every leaf not
    covered by a super cluster: blocks outside complete groups and the tail)
    hold fewer eligible long-range keys for t than the query's budget
    ``sp.budget_at(t)``, so the budget is filled whenever the context holds
    enough keys (the budget is a fixed number of keys per query: mauroscia.it,
    D-LSA paragraph; sysnote.net, "What it changes").  With a third level the
    same walk runs over the top nodes first (``tree2_top`` of them, more
    while the supers under the nodes taken, plus the supers under no top
    node and the uncovered leaves, hold fewer eligible keys than the budget),
    and the super clusters ranked are only those under the top nodes taken
    plus every super cluster not under a top node.
    """
    if idx.params.tree_group <= 0:
        return np.arange(idx.n_bkt, dtype=np.int64)
    need = sp.budget_at(t)

    def sup_weight(s: int) -> int:
        return sum(eligible_count(idx, int(b), t, sp) for b in idx.sup_members[s])

    loose = np.arange(idx.covered_leaves(), idx.n_bkt, dtype=np.int64)
    held = sum(eligible_count(idx, int(b), t, sp) for b in loose)
    sup_ids = np.arange(idx.sup_centroids.shape[0], dtype=np.int64)
    if idx.params.tree2_group > 0:
        loose_sup = np.arange(idx.covered_supers(), len(sup_ids), dtype=np.int64)
        held_top = held + sum(sup_weight(int(s)) for s in loose_sup)
        ts = scores(idx.top_centroids, q)
        top_order = np.lexsort((np.arange(len(ts)), -ts))
        tops = _walk(top_order, sp.tree2_top, held_top, need,
                     lambda n: sum(sup_weight(int(s)) for s in idx.top_members[n]))
        sparts = [idx.top_members[n] for n in tops]
        sparts.append(loose_sup)
        sup_ids = np.sort(np.concatenate(sparts))
    ss = scores(idx.sup_centroids[sup_ids], q)
    order = sup_ids[np.lexsort((sup_ids, -ss))]
    taken = _walk(order, sp.tree_top, held, need, sup_weight)
    parts = [idx.sup_members[s] for s in taken]
    parts.append(loose)
    return np.sort(np.concatenate(parts)) if parts else np.zeros(0, np.int64)


def select(idx: Index, q: np.ndarray, t: int, sp: SelectParams) -> np.ndarray:
    """Sorted key ids attended by the query at position t (t < idx.T).

    Candidate buckets are visited in (score desc, bucket id asc) order; each
    contributes its eligible keys in ascending position until the budget
    (``sp.budget_at(t)``) of long-range keys is held (the last bucket is cut
    at its lowest positions).  The window [t-w+1, t] and the sinks [0, sinks) are added;
    every key is <= t.
    """
    cand = candidates(idx, q, sp, t)
    s = scores(idx.centroids[cand], q)
    order = cand[np.lexsort((cand, -s))]
    picked: List[np.ndarray] = []
    need = sp.budget_at(t)
    for beta in order:
        if need <= 0:
            break
        e = eligible_keys(bucket_keys(idx, int(beta)), t, sp)
        if e.size == 0:
            continue
        take = e[:need]
        picked.append(take)
        need -= take.size
    window = np.arange(max(0, t - sp.window + 1), t + 1, dtype=np.int64)
    sinks = np.arange(0, min(sp.sinks, t + 1), dtype=np.int64)
    allk = np.concatenate(picked + [window, sinks])
    return np.unique(allk)


def dense_select(latk: np.ndarray, q: np.ndarray, t: int, sp: SelectParams) -> np.ndarray:
    """Quadratic comparator: score every long-range key itself, keep the best
    ``sp.budget_at(t)`` by (score desc, position asc), add the window and
    the sinks."""
    lo, hi = sp.sinks, t - sp.window
    keys = np.arange(lo, hi + 1, dtype=np.int64) if hi >= lo else np.zeros(0, np.int64)
    sc = scores(latk[keys], q) if keys.size else np.zeros(0, np.int64)
    best = keys[np.lexsort((keys, -sc))][: sp.budget_at(t)]
    window = np.arange(max(0, t - sp.window + 1), t + 1, dtype=np.int64)
    sinks = np.arange(0, min(sp.sinks, t + 1), dtype=np.int64)
    return np.unique(np.concatenate([best, window, sinks]))


# --------------------------------------------------------------------------
# attention over the selected keys (sysnote.net: the attention itself is
# unchanged, LSA only decides which keys are read)
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (round to nearest, ties to even), as float64:
    the value a bf16 store of x holds.  Rounds x itself, not an intermediate
    float32."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])                  # x = m * 2^e, 0.5 <= |m| < 1
    # 8 significant bits: scale m to [128, 256), round half to even
    out[nz] = np.ldexp(np.round(m * 256.0), e - 8)
    return out


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, Hkv: int,
           scale: Optional[float] = None) -> np.ndarray:
    """Softmax attention of one token over the selected rows.

    q: float64 [Hq][D]; K, V: float64 [n_sel][Hkv][D] (the selected rows).
    Head h uses KV head floor(h * Hkv / Hq).  Returns float64 [Hq][D].
    """
    Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = (K[:, g, :] @ q[h]) * scale
        w = np.exp(logits - logits.max())
        w /= w.sum()
        out[h] = w @ V[:, g, :]
    return out


def attend_lse(q: np.ndarray, K: np.ndarray, V: np.ndarray, Hkv: int,
               scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """attend() and, per head, the natural log of the softmax denominator
    (log-sum-exp of the scaled logits over the selected rows): float64 [Hq]."""
    Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    lse = np.zeros(Hq, dtype=np.float64)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = (K[:, g, :] @ q[h]) * scale
        m = logits.max()
        lse[h] = m + np.log(np.exp(logits - m).sum())
    return attend(q, K, V, Hkv, scale), lse


# --------------------------------------------------------------------------
# backward of the sparse attention over stored selections ("Latent Sparse
# Attention: un indice gerarchico per contesti lunghi", mauroscia.it, N-LSA
# paragraph: training keeps the indices of the selected keys for the backward
# pass).  The selection is discrete and fixed; gradients flow to Q, K and V
# through the softmax attention only.  Per head h (KV head g), with
# s_j = scale * k_j . q_h, p = softmax(s), o_h = sum_j p_j v_j and the
# upstream gradient do_h:
#   dv_j += p_j do_h
#   dp_j  = do_h . v_j
#   ds_j  = p_j (dp_j - sum_k p_k dp_k)
#   dq_h  = scale * sum_j ds_j k_j
#   dk_j += scale * ds_j q_h
# --------------------------------------------------------------------------
def attend_backward(q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, Hkv: int,
                    scale: Optional[float] = None, o: Optional[np.ndarray] = None
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of sum(dO * attend(q, K, V)) for one token.

    q, dO: float64 [Hq][D]; K, V: float64 [n_sel][Hkv][D].  Returns
    (dq [Hq][D], dK [n_sel][Hkv][D], dV [n_sel][Hkv][D]); a row listed twice
    would get the sum of both entries' gradients.  sum_k p_k dp_k equals
    do_h . o_h; given ``o`` (the forward output as a caller stored it, e.g.
    rounded to bf16) that dot product is taken from it instead.
    """
    Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros_like(q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        logits = (K[:, g, :] @ q[h]) * scale
        p = np.exp(logits - logits.max())
        p /= p.sum()
        dV[:, g, :] += np.outer(p, dO[h])
        dp = V[:, g, :] @ dO[h]
        dsum = (p * dp).sum() if o is None else float(dO[h] @ o[h])
        ds = p * (dp - dsum)
        dq[h] = scale * (ds @ K[:, g, :])
        dK[:, g, :] += scale * np.outer(ds, q[h])
    return dq, dK, dV


def sparse_attention_backward(Q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, dO: np.ndarray,
                              rows: Sequence[np.ndarray], Hkv: int, scale: Optional[float] = None,
                              O: Optional[np.ndarray] = None
                              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients for a batch of tokens: token i attends over cache rows rows[i].

    Q, dO: float64 [n][Hq][D]; Kc, Vc: float64 [T][Hkv][D].  Returns
    dQ [n][Hq][D] and dK, dV [T][Hkv][D], where a cache row's gradient is the
    sum over every token that selected it (zero if none did).  ``O``: the
    stored forward outputs (see attend_backward's ``o``), or None.
    """
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(Kc)
    dV = np.zeros_like(Vc)
    for i, r in enumerate(rows):
        r = np.asarray(r, dtype=np.int64)
        dq, dk, dv = attend_backward(Q[i], Kc[r], Vc[r], dO[i], Hkv, scale,
                                     None if O is None else O[i])
        dQ[i] = dq
        np.add.at(dK, r, dk)
        np.add.at(dV, r, dv)
    return dQ, dK, dV
