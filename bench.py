#!/usr/bin/env python3
"""Benchmark of the LSA hot path on one MI355X.

A step is one prefill chunk of one attention layer at the headline shape:
the last 32768 query tokens of a 10*2^20-token context (Flat index, 64-d int8
latents, p=4, blocks of 4096 pooled vectors with 256 buckets, 4 k-means
iterations; GQA 32 query / 8 KV heads, head dim 128, bf16 KV cache held on
the GPU; 4096 long-range + 512 window + 4 sink keys per query).  The step
appends the chunk's keys to the prebuilt index (pooling + clustering of the
two blocks the chunk completes), selects keys for the 32768 queries and runs
the sparse attention.  Inputs are synthetic (lsa_synth) and resident in HBM
before the timed region.

Prints one JSON line.  Extra fields: per-phase times, the attention kernel's
roofline, decode tokens/s (8 sequences of 2^20 keys), full index-build
keys/s, the on-GPU dense per-key scan (the quadratic comparison) and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hierarchical_sparse_attention_lsa_amd as L  # noqa: E402
import lsa_synth as S  # noqa: E402

HBM_PEAK_GBS = 8000.0
INT8_PEAK_OPS = 5.0e15          # dense int8 MFMA, ops/s
ATTN_SRC = os.path.join(ROOT, "hierarchical_sparse_attention_lsa_amd", "csrc", "lsa_attn.hip")
ATTN_KERNEL = "k_attn_grp<128, false>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The measured kernel (the window-sharing attention and the tile code it
# uses) is the part of its source before the decode kernels; counters taken
# on it stay valid while only the code after this marker changes.
ATTN_SRC_END = b"// Decode: split-K attention."


def src_hash(path: str) -> str:
    with open(path, "rb") as f:
        data = f.read()
    cut = data.find(ATTN_SRC_END)
    return hashlib.sha256(data if cut < 0 else data[:cut]).hexdigest()[:16]


def gen_inputs(wl, dev, seq=0, T=None):
    g = S.Synth(wl, seq=seq)
    T = T or wl.T
    latk = g.latk(0, T, device=dev, chunk=1 << 22)
    K = torch.empty((T, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0, chunk=1 << 18)
    g.fill_rows("v", V, 0, chunk=1 << 18)
    return g, latk, K, V


def iparams(wl, cap):
    return L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group,
                         wl.tree_super, wl.tree_iters, cap, wl.tree2_group, wl.tree2_super,
                         wl.tree2_iters)


def attn_algorithmic_bytes(wl, t0, n, cnt: np.ndarray) -> float:
    """Algorithmic HBM bytes of one attention launch over the chunk.

    Long-range rows are counted per query (their reuse is data dependent and
    not credited); window and sink rows form one span for the whole chunk and
    are counted once; plus the index entries read (the long-range part of
    each row and its count), Q and O."""
    row = wl.Hkv * wl.D * 2 * 2                     # K + V bytes per token
    t = np.arange(t0, t0 + n)
    wstart = np.maximum(0, t - wl.window + 1)
    nw = t - wstart + 1
    ns = np.maximum(0, np.minimum(wl.sinks, wstart))
    lr = cnt.astype(np.int64) - nw - ns
    span = (t0 + n - max(0, t0 - wl.window + 1)) + min(wl.sinks, max(0, t0 - wl.window + 1))
    qo = n * wl.Hq * wl.D * 2 * 2
    return float(lr.sum() * row + span * row + lr.sum() * 4 + n * 4 + qo)


def window_span_bytes(wl, t0, n) -> float:
    """K + V bytes of the chunk's window and sink span (read once)."""
    row = wl.Hkv * wl.D * 2 * 2
    span = (t0 + n - max(0, t0 - wl.window + 1)) + min(wl.sinks, max(0, t0 - wl.window + 1))
    return float(span * row)


def _grp_mix(x: np.ndarray) -> np.ndarray:
    """The grouped attention's 32-bit mix (uint32 arithmetic, wrapping)."""
    x = x.astype(np.uint64)
    m = np.uint64(0xFFFFFFFF)
    x = (x * np.uint64(0x9E3779B1)) & m
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x85EBCA6B)) & m
    x ^= x >> np.uint64(13)
    return x


NN_BLOCK = 32768          # queries whose nearest neighbours are searched together


def latent_nn_roots(latq_h: np.ndarray) -> np.ndarray:
    """Host recount of the grouped attention's latent order: each query's
    nearest other query of its block of NN_BLOCK (the j != i maximising
    2 x_i.x_j - |x_j|^2, lowest j of equal scores; float32 holds these
    integers exactly), then the lower index of the mutual pair each query's
    chain of neighbours ends in."""
    x = torch.from_numpy(latq_h.astype(np.float32))
    n = x.shape[0]
    nrm = (x * x).sum(1)
    nn = np.arange(n, dtype=np.int64)
    for base in range(0, n, NN_BLOCK):
        e = min(n, base + NN_BLOCK)
        if e - base < 2:
            continue
        for b0 in range(base, e, 2048):
            b1 = min(e, b0 + 2048)
            s = 2 * x[b0:b1] @ x[base:e].T - nrm[None, base:e]
            r = torch.arange(b1 - b0)
            s[r, r + b0 - base] = -float("inf")
            nn[b0:b1] = base + s.argmax(1).numpy()
    p = nn.copy()
    reach = 1
    while reach < 2 * min(n, NN_BLOCK):
        p = p[p]
        reach *= 2
    return np.minimum(p, nn[p])


def grouped_unions(wl, t0, idx_h: np.ndarray, cnt_h: np.ndarray, latq_h=None):
    """Host recount of the grouped attention's work: queries ordered by the
    first long-range key of their rows, then by the row's MinHash (the
    smallest mix of its pooled-group ids, top 16 bits), then by index -- or,
    with the latent queries, by (first long-range key of the query's
    nearest-neighbour root >> 4, root, index) -- and taken 16/G at a time;
    each group's union is the set of distinct long-range keys of its rows.
    Returns (union rows per group, long-range entries per query)."""
    n = idx_h.shape[0]
    assert n < (1 << 20) - 1, "these orders apply below 2^20 queries"
    t = np.arange(t0, t0 + n)
    wstart = np.maximum(0, t - wl.window + 1)
    lr = cnt_h.astype(np.int64) - (np.maximum(0, np.minimum(wl.sinks, wstart)) + (t - wstart + 1))
    first = np.where(lr > 0, idx_h[:, 0].astype(np.int64), (1 << 28) - 1)
    if latq_h is not None:
        root = latent_nn_roots(latq_h)
        order = np.lexsort((np.arange(n), root, first[root] >> 4))
    else:
        mh = np.array([int(_grp_mix(idx_h[q, :lr[q]].astype(np.uint64) >> np.uint64(2)).min()) >> 16
                       if lr[q] > 0 else 0xFFFF for q in range(n)], dtype=np.int64)
        order = np.lexsort((np.arange(n), mh, first))
    qpw = 16 // (wl.Hq // wl.Hkv)
    unions = []
    for g0 in range(0, n, qpw):
        qs = order[g0:g0 + qpw]
        unions.append(np.unique(np.concatenate([idx_h[q, :lr[q]] for q in qs])).size)
    return np.asarray(unions, dtype=np.int64), lr


def grouped_attn_bytes(wl, t0, n, unions: np.ndarray):
    """Algorithmic HBM bytes of the grouped attention over a chunk.

    walk (k_attn_grp, one launch): every union row's K and V for all KV
    heads, its index entry and mask (5 bytes), the sinks-and-window partials
    (float32 output + max + sum per query head), Q, and the output.
    prepare: the sinks-and-window phase reads the chunk's window span (and
    sinks) once, Q, and writes the partials; the sort and union kernels read
    the rows' long-range parts and write the unions (counted as union rows x
    5 bytes written; the row reads are of the same order and left out)."""
    row = wl.Hkv * wl.D * 2 * 2
    heads = n * wl.Hq
    partials = heads * (wl.D + 2) * 4
    q_bytes = heads * wl.D * 2
    o_bytes = heads * wl.D * 2
    u = int(unions.sum())
    walk = u * row + u * 5 + partials + q_bytes + o_bytes + n * 4 + len(unions) * 4
    span = (t0 + n - max(0, t0 - wl.window + 1)) + min(wl.sinks, max(0, t0 - wl.window + 1))
    prepare = span * row + q_bytes + partials + u * 5
    return float(walk), float(prepare)


def bench_prefill(args, dev):
    wl = S.WORKLOADS[args.config]
    n = wl.chunk
    t0 = wl.T - n
    log(f"[bench] generating {wl.name}: T={wl.T} keys, KV {2 * wl.T * wl.Hkv * wl.D * 2 / 2**30:.1f} GiB")
    tg = time.time()
    g, latk, K, V = gen_inputs(wl, dev)
    pos = torch.arange(t0, wl.T, dtype=torch.int64)
    latq = g.latq_rows(pos.to(dev), device=dev)
    q = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    g.fill_rows("q", q, t0)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - tg:.1f}s")

    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, 0, 0, wl.tree2_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    ix = L.LsaIndex(iparams(wl, wl.T), dev)

    # full index build over the whole context (reported as keys/s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    build_ms = []
    for _ in range(3):
        ev[0].record()
        ix.build(latk)
        ev[1].record()
        torch.cuda.synchronize()
        build_ms.append(ev[0].elapsed_time(ev[1]))
    # prebuilt index of the context before the chunk
    ix.build(latk[:t0])
    torch.cuda.synchronize()
    snap = ix.snapshot()

    idx = torch.empty((n, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((n,), dtype=torch.int32, device=dev)
    out = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    qpos = torch.arange(t0, wl.T, dtype=torch.int32, device=dev)
    lk_chunk = latk[t0:]
    sel_ws = torch.empty(max(L.workspace_bytes(L.binding.OP_SELECT, ix.params, sp, None, n), 256),
                         dtype=torch.uint8, device=dev)
    grp_ws = torch.empty(L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap, n),
                         dtype=torch.uint8, device=dev)

    # one step: append the chunk, select, attend (grouped: prepare, then the
    # long-range walk); every call on torch's current stream, where the events
    # are recorded.  The queries are grouped by their latent neighbours, or by
    # their rows on a three-level Tree index (as lsa_prefill_chunk does).
    glat = latq if wl.tree2_group == 0 else None

    def step(evs=None):
        ix.restore(snap)
        if evs: evs[0].record()
        ix.append(lk_chunk)
        if evs: evs[1].record()
        ix.select(latq, qpos, sp, idx=idx, cnt=cnt, ws=sel_ws)
        if evs: evs[2].record()
        L.sparse_attn_grouped(q, K, V, idx, cnt, t0, sp, ap, ws=grp_ws, part="prepare", latq=glat)
        if evs: evs[3].record()
        L.sparse_attn_grouped(q, K, V, idx, cnt, t0, sp, ap, out=out, ws=grp_ws, part="walk")
        if evs: evs[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ph4 = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])
    ph = np.stack([ph4[:, 0], ph4[:, 1], ph4[:, 2] + ph4[:, 3]], axis=1)
    ms_per_step = wall * 1e3 / args.steps

    # context: the ungrouped window-sharing kernel on the same rows
    out_w = torch.empty_like(out)
    L.sparse_attn_window(q, K, V, idx, cnt, t0, sp, ap, out=out_w)
    ew = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    win_ms = []
    for _ in range(2):
        ew[0].record()
        L.sparse_attn_window(q, K, V, idx, cnt, t0, sp, ap, out=out_w)
        ew[1].record()
        torch.cuda.synchronize()
        win_ms.append(ew[0].elapsed_time(ew[1]))
    del out_w

    # the fused entry point gives the same selection and output
    ix.restore(snap)
    idx2 = torch.empty_like(idx)
    cnt2 = torch.empty_like(cnt)
    out2 = ix.prefill_chunk(lk_chunk, latq, q, K, V, sp, ap, idx=idx2, cnt=cnt2)
    torch.cuda.synchronize()
    fused_same = bool(torch.equal(idx2, idx) and torch.equal(cnt2, cnt) and
                      torch.equal(out2.view(torch.int16), out.view(torch.int16)))

    cnt_h = cnt.cpu().numpy()
    unions, lr = grouped_unions(wl, t0, idx.cpu().numpy(), cnt_h,
                                glat.cpu().numpy() if glat is not None else None)
    walk_bytes, prep_bytes = grouped_attn_bytes(wl, t0, n, unions)
    attn_ms = float(ph4[:, 3].mean())                  # the long-range walk: one launch
    per_query = attn_algorithmic_bytes(wl, t0, n, cnt_h)
    # the walk's share of the per-query accounting: everything but the
    # window and sink span, which the prepare half reads
    walk_pq = per_query - window_span_bytes(wl, t0, n)
    res = {
        "wl": wl, "t0": t0, "n": n, "ms_per_step": ms_per_step, "phase_ms": ph.mean(0).tolist(),
        "step_event_ms": {"median": float(np.median(ph.sum(1))), "min": float(ph.sum(1).min()),
                          "attention_median": float(np.median(ph[:, 2])),
                          "attention_min": float(ph[:, 2].min())},
        "attn_ms": attn_ms, "attn_bytes": walk_pq, "achieved_gbs": walk_pq / (attn_ms * 1e-3) / 1e9,
        "attn_union_bytes": walk_bytes, "union_gbs": walk_bytes / (attn_ms * 1e-3) / 1e9,
        "attn_phase_bytes": walk_bytes + prep_bytes, "attn_phase_bytes_per_query": per_query,
        "grouped": {"prepare_ms": float(ph4[:, 2].mean()), "walk_ms": attn_ms,
                    "union_rows": int(unions.sum()), "long_range_entries": int(lr.sum()),
                    "union_fraction": float(unions.sum() / max(1, lr.sum())),
                    "groups": int(len(unions)), "prepare_algorithmic_bytes": prep_bytes,
                    "ungrouped_window_kernel_ms": float(np.median(win_ms)),
                    "per_query_algorithmic_bytes": per_query,
                    "per_query_bytes_over_attention_phase_gbs":
                        per_query / (float(ph[:, 2].mean()) * 1e-3) / 1e9},
        "build_ms": float(np.median(build_ms)), "fused_same": fused_same,
        "cnt_mean": float(cnt_h.mean()), "g": g, "latk": latk, "latq": latq, "idx": idx,
        "cnt": cnt, "out": out, "K": K, "V": V, "q": q, "ix": ix, "snap": snap, "sp": sp,
    }
    return res


def bench_tree_same_data(res, dev, steps, warmup, name="tree_10m"):
    """The two-level Tree workload on the Flat step's own data (the Tree
    workloads share the 10M context, chunk, Q/K/V and latents): the same
    append + select + attention step on a Tree index, with the number of
    keys each query selected."""
    wl = S.WORKLOADS[name]
    t0, n = res["t0"], res["n"]
    assert wl.T == res["wl"].T and wl.chunk == n
    ix = L.LsaIndex(iparams(wl, wl.T), dev)
    ix.build(res["latk"][:t0])
    torch.cuda.synchronize()
    snap = ix.snapshot()
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, 0, 0, wl.tree2_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    idx = torch.empty((n, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((n,), dtype=torch.int32, device=dev)
    out = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    qpos = torch.arange(t0, wl.T, dtype=torch.int32, device=dev)
    ws = torch.empty(max(L.workspace_bytes(L.binding.OP_SELECT, ix.params, sp, None, n), 256),
                     dtype=torch.uint8, device=dev)
    gws = torch.empty(L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap, n), dtype=torch.uint8,
                      device=dev)
    lk_chunk = res["latk"][t0:]
    glat = res["latq"] if wl.tree2_group == 0 else None     # as lsa_prefill_chunk orders them

    def step(e=None):
        ix.restore(snap)
        if e: e[0].record()
        ix.append(lk_chunk)
        if e: e[1].record()
        ix.select(res["latq"], qpos, sp, idx=idx, cnt=cnt, ws=ws)
        if e: e[2].record()
        L.sparse_attn_grouped(res["q"], res["K"], res["V"], idx, cnt, t0, sp, ap, out=out, ws=gws,
                              latq=glat)
        if e: e[3].record()

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / steps
    ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                   for e in evs]).mean(0)
    cnt_h = cnt.cpu().numpy()
    unions, _ = grouped_unions(wl, t0, idx.cpu().numpy(), cnt_h,
                               glat.cpu().numpy() if glat is not None else None)
    walk_b, prep_b = grouped_attn_bytes(wl, t0, n, unions)
    del idx, out, ws, gws
    return {"workload": name, "index": f"Flat leaves + Tree G={wl.tree_group} S={wl.tree_super} "
                                        f"R={wl.tree_top} (walk fills the budget)",
            "ms_per_step": ms, "queries_per_s": n / (ms * 1e-3),
            "phases_ms": {"append": float(ph[0]), "select": float(ph[1]), "attention": float(ph[2])},
            "selected_keys_per_query": {"mean": float(cnt_h.mean()), "min": int(cnt_h.min()),
                                        "budget": wl.max_sel},
            "attention_phase_frac": (walk_b + prep_b) / (ph[2] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "union_fraction": float(unions.sum()) / float(res["grouped"]["long_range_entries"])}


def bench_other_config(name, args, dev):
    """The same prefill step (prebuilt index, append, select, grouped
    attention) on another Flat workload, with its roofline fractions: the
    walk against the HBM peak (per-query and union bytes), the step against
    its layer roof, and the index build against its roof."""
    a = argparse.Namespace(**vars(args))
    a.config = name
    r = bench_prefill(a, dev)
    wl = r["wl"]
    ms = r["ms_per_step"]
    roof = layer_roof_ms(wl, r, r["attn_phase_bytes_per_query"])
    out = {"workload": name, "context_tokens": wl.T, "chunk_queries": r["n"],
           "attention": f"GQA {wl.Hq}/{wl.Hkv} D={wl.D} bf16",
           "select": f"{wl.budget}+{wl.window}+{wl.sinks}",
           "ms_per_step": ms, "queries_per_s": r["n"] / (ms * 1e-3),
           "phases_ms": {"append": r["phase_ms"][0], "select": r["phase_ms"][1],
                         "attention": r["phase_ms"][2]},
           "selected_keys_per_query": r["cnt_mean"],
           "union_fraction": r["grouped"]["union_fraction"],
           "walk_ms": r["attn_ms"],
           "walk_frac_per_query_bytes": r["achieved_gbs"] / HBM_PEAK_GBS,
           "walk_frac_union_bytes": r["union_gbs"] / HBM_PEAK_GBS,
           "layer": {"roof_ms": roof, "frac": roof / ms},
           "index_build": {"keys": wl.T, "ms": r["build_ms"],
                           "keys_per_s": wl.T / (r["build_ms"] * 1e-3),
                           "roof_ms": build_roof_ms(wl), "frac": build_roof_ms(wl) / r["build_ms"]},
           "fused_entry_point_identical": r["fused_same"]}
    del r
    torch.cuda.empty_cache()
    return out


def measured_copy_gbs(dev, nbytes=2 << 30):
    """Read + write bandwidth of a plain device copy (torch), for context."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(3):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (min(ts) * 1e-3) / 1e9


def layer_roof_ms(wl, res, attn_bytes):
    """Roofline time of the whole chunk step: the attention's bytes at the HBM
    peak plus the query x centroid scoring at the int8 MFMA peak (append and
    the rest of the selection are latency terms with no bandwidth floor of
    note)."""
    n_bkt = (wl.T // wl.pool // wl.block) * wl.buckets
    score_ops = 2.0 * res["n"] * n_bkt * 64
    return attn_bytes / (HBM_PEAK_GBS * 1e9) * 1e3 + score_ops / INT8_PEAK_OPS * 1e3


def build_roof_ms(wl) -> float:
    """Roofline of a full index build over T keys: read the latents, write the
    pooled vectors, centroids, member lists and bucket descriptors (HBM), and
    the k-means distance products at the int8 MFMA peak; the larger bounds."""
    n_pool = wl.T // wl.pool
    n_bkt = n_pool // wl.block * wl.buckets
    nbytes = wl.T * 64 + n_pool * 64 + n_bkt * 64 + n_pool * 4 + n_bkt * 16
    ops = 2.0 * n_pool * wl.buckets * 64 * wl.iters
    return max(nbytes / (HBM_PEAK_GBS * 1e9), ops / INT8_PEAK_OPS) * 1e3


def select_roof_ms(wl, n) -> float:
    """Roofline of the chunk's selection: every (query, bucket) score at the
    int8 MFMA peak, plus writing the selected rows at the HBM peak."""
    n_bkt = (wl.T // wl.pool // wl.block) * wl.buckets
    return (2.0 * n * n_bkt * 64 / INT8_PEAK_OPS + n * wl.max_sel * 4 / (HBM_PEAK_GBS * 1e9)) * 1e3


def dense_roof_ms(wl, t0, n) -> float:
    """Roofline of the dense per-key comparator over the chunk: every
    (query, long-range key) latent product at the int8 MFMA peak."""
    t = np.arange(t0, t0 + n, dtype=np.float64)
    keys = np.maximum(0.0, t - wl.window - wl.sinks + 1)
    return float(2.0 * 64 * keys.sum() / INT8_PEAK_OPS * 1e3)


def bench_dense(res, dev):
    """Quadratic comparison: every long-range key of the 10M context scored on
    its own latent for all of the chunk's queries (one thresholded int8-MFMA
    scan of the latents plus an exact top-budget per query), with the same
    selection rule (singleton buckets of p = 1)."""
    wl, t0, n = res["wl"], res["t0"], res["n"]
    sp = res["sp"]
    qpos = torch.arange(t0, t0 + n, dtype=torch.int32, device=dev)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DENSE, None, sp, None, n), dtype=torch.uint8, device=dev)
    L.dense_select(res["latk"], res["latq"][:64].contiguous(), qpos[:64].contiguous(), sp)   # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    idx, cnt = L.dense_select(res["latk"], res["latq"], qpos, sp, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # the rows are the rule's: each query holds budget + window + sinks keys
    full = bool((cnt == sp.max_sel).all().item())
    del idx, cnt, ws
    torch.cuda.empty_cache()
    roof = dense_roof_ms(wl, t0, n)
    return {"queries": n, "ms_per_chunk": ms, "rows_full": full,
            "roofline": {"bound": "mfma int8", "roof_ms_per_chunk": roof, "frac": roof / ms},
            "note": "dense per-key int8 scan + exact top-B over all long-range keys, same "
                    "selection rule (p=1 singleton buckets)"}


def bench_full_prefill(args, dev, data=None):
    """Every chunk of the context through lsa_prefill_chunk, the index grown
    chunk by chunk from empty: the whole prefill of one layer (a per-layer
    time-to-first-token analogue).  Only the fused calls are timed; the next
    chunk's Q and latent queries are generated outside the timed regions.
    `data`: the workload's (generator, latents, K, V) when already on the
    device."""
    wl = S.WORKLOADS[args.config]
    n = wl.chunk
    nchunks = wl.T // n
    log(f"[full] {wl.name}: {nchunks} chunks of {n} queries")
    g, latk, K, V = data if data is not None else gen_inputs(wl, dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    ix = L.LsaIndex(iparams(wl, wl.T), dev)
    q = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    out = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_PREFILL, ix.params, sp, ap, n), dtype=torch.uint8,
                     device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for c in range(nchunks):
        t0 = c * n
        latq = g.latq_rows(torch.arange(t0, t0 + n, device=dev), device=dev)
        g.fill_rows("q", q, t0)
        torch.cuda.synchronize()
        e0.record()
        ix.prefill_chunk(latk[t0:t0 + n], latq, q, K, V, sp, ap, out=out, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        if c % 32 == 0 or c == nchunks - 1:
            log(f"[full] chunk {c}: {times[-1]:.2f} ms")
    t = np.array(times)
    return {"workload": wl.name, "context_tokens": wl.T, "chunks": nchunks, "chunk_queries": n,
            "total_s": float(t.sum() / 1e3), "queries_per_s": float(wl.T / (t.sum() / 1e3)),
            "chunk_ms": {"first": float(t[0]), "median": float(np.median(t)), "last": float(t[-1]),
                         "max": float(t.max())}}


def bench_train(args, dev, steps=3, warmup=1):
    """One attention layer's training step at 128k context, every position a
    query: index build over all keys, selection, forward with log-sum-exp
    (the grouped attention), backward (dQ, dK, dV) from a synthetic upstream
    gradient.  Phases are timed with events on the stream the kernels run
    on."""
    wl = S.WORKLOADS["train_128k"]
    T = wl.T
    log(f"[train] generating {wl.name}: T={T}, every position a query")
    g, latk, K, V = gen_inputs(wl, dev)
    pos = torch.arange(0, T, device=dev)
    latq = g.latq_rows(pos, device=dev)
    q = torch.empty((T, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    do = torch.empty_like(q)
    g.fill_rows("q", q, 0)
    g.fill_rows("do", do, 0)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    ix = L.LsaIndex(iparams(wl, T), dev)
    qpos = pos.to(torch.int32)
    idx = torch.empty((T, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((T,), dtype=torch.int32, device=dev)
    out = torch.empty((T, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, wl.Hq), dtype=torch.float32, device=dev)
    dq = torch.empty((T, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    dk = torch.empty((T, wl.Hkv, wl.D), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    sel_ws = torch.empty(L.workspace_bytes(L.binding.OP_SELECT, ix.params, sp, None, T),
                         dtype=torch.uint8, device=dev)
    bwd_ws = torch.empty(L.workspace_bytes(L.binding.OP_ATTN_BWD, ix.params, sp, ap, T),
                         dtype=torch.uint8, device=dev)
    grp_ws = torch.empty(L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap, T),
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def step():
        ev[0].record()
        ix.build(latk)
        ev[1].record()
        ix.select(latq, qpos, sp, idx=idx, cnt=cnt, ws=sel_ws)
        ev[2].record()
        L.sparse_attn_grouped(q, K, V, idx, cnt, 0, sp, ap, out=out, ws=grp_ws, lse=lse, latq=latq)
        ev[3].record()
        L.sparse_attn_bwd(ix, q, K, V, idx, cnt, 0, sp, ap, out, lse, do, dq=dq, dk=dk, dv=dv,
                          ws=bwd_ws, latq=latq)
        ev[4].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ph = np.zeros(4)
    for _ in range(steps):
        step()
        torch.cuda.synchronize()
        ph += [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    ph /= steps
    cnt_h = cnt.cpu().numpy()
    fwd_bytes = attn_algorithmic_bytes(wl, 0, T, cnt_h)
    total = float(ph.sum())
    res = {"workload": wl.name, "context_tokens": T, "queries": T,
           "ms_per_step": total, "tokens_per_s": T / (total * 1e-3),
           "phases_ms": {"index_build": float(ph[0]), "select": float(ph[1]),
                         "forward": float(ph[2]), "backward": float(ph[3])},
           # per-query accounting (every query's rows counted): the grouped
           # forward reads less, so this rate can pass the HBM peak
           "forward_per_query_bytes_gbs": fwd_bytes / (ph[2] * 1e-3) / 1e9,
           "forward_per_query_bytes": fwd_bytes,
           "selected_keys_per_query": float(cnt_h.mean())}
    log(f"[train] step {total:.1f} ms: build {ph[0]:.2f}, select {ph[1]:.2f}, forward {ph[2]:.2f}, "
        f"backward {ph[3]:.2f} ms; forward {res['forward_per_query_bytes_gbs']:.0f} GB/s per-query accounting")
    return res


def bench_decode(args, dev, wl=None):
    wl = wl or S.WORKLOADS["decode_1m"]
    cap = wl.T + wl.steps
    log(f"[bench] decode: {wl.nseq} sequences x {wl.T} keys, {wl.steps} steps")
    ixs, lat, gens = [], [], []
    K = torch.empty((wl.nseq, cap, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for i in range(wl.nseq):
        g = S.Synth(wl, seq=i)
        gens.append(g)
        lk = g.latk(0, cap, device=dev, chunk=1 << 22)
        lat.append(lk)
        g.fill_rows("k", K[i], 0, chunk=1 << 18)
        g.fill_rows("v", V[i], 0, chunk=1 << 18)
        ix = L.LsaIndex(iparams(wl, cap), dev)
        ix.build(lk[:wl.T])
        ixs.append(ix)
    steps = wl.steps
    new_pos = torch.arange(wl.T, wl.T + steps, dtype=torch.int64, device=dev)
    lk_new = torch.stack([lat[i][wl.T:wl.T + steps] for i in range(wl.nseq)], 1).contiguous()
    lq = torch.stack([gens[i].latq_rows(new_pos, device=dev) for i in range(wl.nseq)], 1).contiguous()
    qs = torch.stack([gens[i].q_rows(new_pos, device=dev) for i in range(wl.nseq)], 1).contiguous()
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top if wl.tree_group else 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    out = torch.empty((wl.nseq, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    wsb = L.workspace_bytes(L.binding.OP_DECODE, ixs[0].params, sp, ap, wl.nseq)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    snaps = [ix.snapshot() for ix in ixs]
    torch.cuda.synchronize()

    def run():
        for s in range(steps):
            L.decode_step(ixs, lk_new[s], lq[s], qs[s], K, V, cap, sp, ap, out=out, ws=ws)

    run()                       # warm-up pass
    torch.cuda.synchronize()
    for ix, sn in zip(ixs, snaps):
        ix.restore(sn)
    t = time.perf_counter()
    run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t
    # step roofline: the selected K/V rows of the last step plus every centroid scored,
    # at the HBM peak (the kernels' launches and their ramps are what the rest is)
    _, cnt = L.decode_selection(ws, wl.nseq, sp)
    kv_bytes = int(cnt.sum().item()) * wl.Hkv * wl.D * 2 * 2
    cent_bytes = sum(ix.info().n_bkt for ix in ixs) * 64
    step_bytes = kv_bytes + cent_bytes
    ms = dt * 1e3 / steps
    roof_ms = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    return {"sequences": wl.nseq, "context": wl.T, "steps": steps,
            "index": f"Tree G={wl.tree_group} S={wl.tree_super} R={wl.tree_top}" if wl.tree_group else "Flat",
            "ms_per_step": ms, "tokens_per_s": wl.nseq * steps / dt,
            "roofline": {"bound": "hbm", "algorithmic_bytes_per_step": step_bytes,
                         "roof_ms": roof_ms, "frac": roof_ms / ms,
                         "note": "selected K/V rows of every sequence + centroids scored, at the "
                                 "8 TB/s peak, against the whole step (four kernels)"}}


def cpu_baseline(res, workers_pool, n_sample=512):
    """The oracle, timed on host cores on a bounded sample of the same workload."""
    import oracle as O
    from oracle.parallel_build import build_cache_parallel
    from threadpoolctl import threadpool_limits
    wl, t0, n = res["wl"], res["t0"], res["n"]
    g = S.Synth(wl)
    tb = time.time()
    cache0, latk_h = build_cache_parallel(wl.name, t0, workers_pool)   # untimed: prebuilt context
    log(f"[bench] oracle prebuilt index ({t0} keys) in {time.time() - tb:.1f}s")
    # timed: the chunk's index update (pool + cluster the two blocks it completes)
    latk_chunk = g.latk(t0, wl.T).numpy()
    latk_all = np.concatenate([latk_h, latk_chunk])
    params = O.IndexParams(wl.pool, wl.block, wl.buckets, wl.iters)
    # every timed leg runs on one host thread (NumPy's BLAS limited to one
    # thread), so the figure is per core and `cores` is exact
    limit = threadpool_limits(limits=1)
    ts = time.perf_counter()
    P = O.pool(latk_all[t0 - (t0 % (wl.pool * wl.block)):], wl.pool)
    b0 = t0 // (wl.pool * wl.block)
    nb = wl.T // (wl.pool * wl.block) - b0
    blk = []
    for b in range(nb):
        blk.append(O.kmeans(P[b * wl.block:(b + 1) * wl.block], wl.buckets, wl.iters))
    t_update = time.perf_counter() - ts
    cache = dict(cache0)
    for b in range(nb):
        cache[("blk", b0 + b)] = blk[b]
    full = O.build_index(latk_all, wl.T, params, cache)
    # timed: selection + attention for a sample of the chunk's queries
    sel_i = np.unique(np.linspace(0, n - 1, n_sample).round().astype(np.int64))
    positions = (t0 + sel_i).tolist()
    lq = g.latq_rows(torch.tensor(positions)).numpy()
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    m = len(positions)
    sels, t_sel = [], 0.0
    for i, t in enumerate(positions):
        ts = time.perf_counter()
        sels.append(O.select(full, lq[i], t, osp))
        t_sel += time.perf_counter() - ts
        if (i + 1) % 128 == 0:
            log(f"[bench] cpu oracle: {i + 1}/{m} selections, {t_sel:.1f}s")
    limit.restore_original_limits()
    qh = O.bf16_to_f64(g.q_rows(torch.tensor(positions)).view(torch.int16).numpy())
    # the selected K/V rows are generated batch by batch outside the timed
    # region (with every host thread), the attention timed on one thread
    outs, t_att = [], 0.0
    for k0 in range(0, m, 32):
        kv = []
        for s in sels[k0:k0 + 32]:
            rows = torch.from_numpy(s)
            kv.append((O.bf16_to_f64(g.k_rows(rows).view(torch.int16).numpy()),
                       O.bf16_to_f64(g.v_rows(rows).view(torch.int16).numpy())))
        limit = threadpool_limits(limits=1)
        ts = time.perf_counter()
        outs += [O.attend(qh[k0 + j], kv[j][0], kv[j][1], wl.Hkv) for j in range(len(kv))]
        t_att += time.perf_counter() - ts
        limit.restore_original_limits()
        del kv
        if (k0 // 32) % 4 == 3 or k0 + 32 >= m:
            log(f"[bench] cpu oracle: {min(k0 + 32, m)}/{m} attention rows, {t_att:.1f}s")
    t_step = t_update + (t_sel + t_att) * n / m
    # parity of the same sample against the GPU's timed step, and of the
    # float32 output of the same kernel (the one the 2e-3 bar applies to)
    idx, cnt = res["idx"].cpu().numpy(), res["cnt"].cpu().numpy()
    same = sum(int(np.array_equal(np.sort(idx[i, :cnt[i]]), sels[j])) for j, i in enumerate(sel_i))
    o = res["out"].float().cpu().numpy()[sel_i]
    ref = np.stack(outs)
    err = float(np.abs(o - ref).max() / np.abs(ref).max())
    ap32 = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    o32 = L.sparse_attn_grouped(res["q"], res["K"], res["V"], res["idx"], res["cnt"], t0, res["sp"], ap32)
    o32 = o32[torch.from_numpy(sel_i).to(o32.device)].cpu().numpy().astype(np.float64)
    err32 = float(np.abs(o32 - ref).max() / np.abs(ref).max())
    per_th = np.abs(o32 - ref).max(-1) / np.abs(ref).max(-1)        # per (token, head)
    return {
        "value": n / t_step, "unit": "queries/s", "cores": 1, "kind": "oracle",
        "sample": f"chunk index update (2 blocks) timed in full; select + attention timed on "
                  f"{m} of {n} chunk queries and scaled to the chunk; prebuilt context index "
                  f"built untimed",
        "host": host_info(),
        "threads": "every timed leg on one thread (Python loops; NumPy BLAS limited to 1 thread)",
        "timed_s": t_update + t_sel + t_att,
        "timed_legs_s": {"index_update": t_update, "select": t_sel, "attention": t_att},
        # the timed step stores bf16, whose rounding alone may reach the unit
        # roundoff 2^-8 of the largest output; the float32 output of the same
        # kernel is held to 2e-3 by the parity tests
        "parity_sample": {"queries": m, "selections_bit_exact": same,
                          "attn_f32_normwise_err": err32, "bar": 2e-3,
                          "bar_applies_to": "the float32 output of the same kernel (out_f32 = 1)",
                          "attn_f32_max_err_per_token_head": float(per_th.max()),
                          "attn_bf16_normwise_err": err, "bf16_unit_roundoff": 2.0 ** -8},
    }


def host_info():
    """The host the oracle ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


CALIB_BYTES = 2 << 30


def profile_run(args, dev):
    """One prefill step (the timed kernels) and a plain 2 GiB device copy whose
    HBM bytes are known, for rocprofv3 counter runs."""
    args.steps, args.warmup = 1, 0
    res = bench_prefill(args, dev)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[profile] prefill step {res['ms_per_step']:.2f} ms; calibration copy of {CALIB_BYTES} bytes done")


# Counter passes of `bench.py --profile` (one rocprofv3 --pmc run each; the
# per-block limits allow these groupings): MFMA work and busy cycles, DRAM
# requests at the L2's memory interface, and the FETCH_SIZE / WRITE_SIZE
# pair.  The summary divides each by what the same counter reads for the
# 2 GiB calibration copy at the end of the run.
PMC_PASSES = {
    "mfma": ["SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_WAVES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "dram": ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum",
             "TCC_EA0_RDREQ_32B_sum"],
    "fetch": ["FETCH_SIZE", "TCC_HIT_sum"],
    "write": ["WRITE_SIZE", "TCC_MISS_sum", "TCC_EA0_WRREQ_64B_sum"],
}
N_SIMD = 1024                    # 256 CUs x 4 SIMDs
# (label, kernel-name substring) of the kernels the prefill summary reports
PREFILL_KERNELS = [("attention", ATTN_KERNEL),
                   ("attention: sinks and window", "k_attn_swin<128>"),
                   ("attention: unions", "k_grp_union<"),
                   ("attention: latent neighbours", "k_grp_nn("), ("select: scan", "k_scan<"),
                   ("select: resolve", "k_resolve("), ("index: k-means", "k_kmeans("),
                   ("index: pool", "k_pool("), ("calibration copy", "__amd_rocclr_copyBuffer")]


def _pmc_dispatches(path):
    """{dispatch id: (kernel name, grid size, {counter: value})}; the values of
    a counter's dimension instances are summed."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        name, c, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
        ent = out.setdefault(d, (name, int(r["Grid_Size"]), {}))
        vals = ent[2]
        vals[c] = vals.get(c, 0.0) + v
    return out


def _largest(disp, key):
    """Counters of the largest-grid (then last) dispatch whose name contains key."""
    best = None
    for d, (name, grid, vals) in disp.items():
        if key in name and (best is None or (grid, d) >= best[0]):
            best = ((grid, d), vals)
    return None if best is None else (best[0][0], best[1])


def _trace_avg_ms(trace_csv, key, grid, longest=False):
    """Average duration (ms) of the kernel-trace dispatches of that name and
    grid (or the longest of them: the runtime's copy kernel launches the same
    grid for copies of every size, and only the calibration copy counts)."""
    import csv
    ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6
          for r in csv.DictReader(open(trace_csv))
          if key in r["Kernel_Name"]
          and int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) == grid]
    if longest and ds:
        return max(ds), 1
    return (sum(ds) / len(ds), len(ds)) if ds else (None, 0)


def _agent(pdir):
    """(SIMD count, XCD count) of the profiled GPU from rocprofv3's agent table."""
    import csv
    for r in csv.DictReader(open(os.path.join(pdir, "mfma", "run_agent_info.csv"))):
        if r.get("Name", "").startswith("gfx"):
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    return N_SIMD, 8


def summarize_prefill(args):
    """profiles/prefill_flat_10m_rocprof.md and profiles/attn_traffic.json from
    `bench.py --profile` runs: a kernel trace and the PMC_PASSES counter runs.

    --summarize-prefill DIR COMMAND, DIR holding trace/, mfma/, dram/, fetch/
    and write/ (rocprofv3 -d DIR/<pass> -o run)."""
    pdir, command = args.summarize_prefill
    trace_csv = os.path.join(pdir, "trace", "run_kernel_trace.csv")
    passes = {k: _pmc_dispatches(os.path.join(pdir, k, "run_counter_collection.csv")) for k in PMC_PASSES}
    copy = {k: _largest(v, "__amd_rocclr_copyBuffer") for k, v in passes.items()}
    cal = {
        "dram_rd": CALIB_BYTES / (copy["dram"][1]["TCC_EA0_RDREQ_DRAM_32B_sum"] * 32),
        "dram_wr": CALIB_BYTES / (copy["dram"][1]["TCC_EA0_WRREQ_DRAM_sum"] * 64),
        "fetch": CALIB_BYTES / (copy["fetch"][1]["FETCH_SIZE"] * 1024),
        "write": CALIB_BYTES / (copy["write"][1]["WRITE_SIZE"] * 1024),
    }
    n_simd, n_xcd = _agent(pdir)
    rows, kern = [], {}
    for label, key in PREFILL_KERNELS:
        got = {k: _largest(v, key) for k, v in passes.items()}
        if any(g is None for g in got.values()):
            continue
        grid = got["mfma"][0]
        ms, calls = _trace_avg_ms(trace_csv, key, grid, longest=key.startswith("__amd_rocclr"))
        m, dr, fe, wr = (got[k][1] for k in ("mfma", "dram", "fetch", "write"))
        cycles = m["GRBM_GUI_ACTIVE"] / n_xcd          # the counter sums the XCDs' cycles
        k = {
            "grid": grid, "trace_avg_ms": ms, "trace_calls": calls,
            "int8_ops": m["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512,
            "bf16_flops": m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
            "mfma_busy_frac": m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * n_simd) if cycles else None,
            "valu_insts": m["SQ_INSTS_VALU"],
            "dram_read_bytes": dr["TCC_EA0_RDREQ_DRAM_32B_sum"] * 32 * cal["dram_rd"],
            "dram_write_bytes": dr["TCC_EA0_WRREQ_DRAM_sum"] * 64 * cal["dram_wr"],
            "fetch_bytes": fe["FETCH_SIZE"] * 1024 * cal["fetch"],
            "write_bytes": wr["WRITE_SIZE"] * 1024 * cal["write"],
            "l2_hit_frac": fe["TCC_HIT_sum"] / max(1.0, fe["TCC_HIT_sum"] + wr["TCC_MISS_sum"]),
        }
        kern[label] = k
        gbs = (k["dram_read_bytes"] + k["dram_write_bytes"]) / (ms * 1e-3) / 1e9 if ms else float("nan")
        rows.append(f"| {label} | `{key}` | {grid} | {ms:.4f} | {k['int8_ops'] / 1e9:.1f} | "
                    f"{k['bf16_flops'] / 1e12:.3f} | {100 * (k['mfma_busy_frac'] or 0):.1f}% | "
                    f"{k['dram_read_bytes'] / 1e9:.3f} | {k['dram_write_bytes'] / 1e9:.3f} | {gbs:.0f} | "
                    f"{(k['fetch_bytes'] + k['write_bytes']) / 1e9:.3f} | {100 * k['l2_hit_frac']:.1f}% |")
    import csv
    stats = list(csv.DictReader(open(os.path.join(pdir, "trace", "run_kernel_stats.csv"))))
    lines = ["# rocprofv3: LSA prefill step, Flat 10M (T = 10*2^20, 32768 queries, GQA 32/8, D = 128)", "",
             "Commands (from the repository root; each pass is its own run):", "", "```", command, "```", "",
             "## Kernel time (kernel trace, all dispatches of the run: 3 full builds, the prebuilt",
             "index, one step, the calibration copy)", "",
             "| kernel | calls | average ms | total ms |", "|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        if "lsa" not in r["Name"]:
            continue
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} |")
    lines += ["", "## Counters per dispatch (largest-grid dispatch of each kernel: the full 10M build for",
              "k-means and pooling, the 32768-query step for the rest)", "",
              "* int8 ops / bf16 flops: `SQ_INSTS_VALU_MFMA_MOPS_I8 / _BF16` x 512.",
              f"* MFMA busy: `SQ_VALU_MFMA_BUSY_CYCLES` (summed over SIMDs) / (`GRBM_GUI_ACTIVE` / {n_xcd} XCDs "
              f"x {n_simd} SIMDs); `GRBM_GUI_ACTIVE` arrives summed over the XCDs.",
              "* DRAM read / write: `TCC_EA0_RDREQ_DRAM_32B_sum` x 32 B and `TCC_EA0_WRREQ_DRAM_sum` x 64 B, "
              "each times its calibration factor; GB/s uses the trace's average duration.",
              "* FETCH+WRITE: `FETCH_SIZE` and `WRITE_SIZE` (KiB) times their calibration factors.",
              f"* Calibration: the 2 GiB device copy reads {copy['dram'][1]['TCC_EA0_RDREQ_DRAM_32B_sum']:.0f} "
              f"32-byte DRAM requests (factor {cal['dram_rd']:.5f}), writes "
              f"{copy['dram'][1]['TCC_EA0_WRREQ_DRAM_sum']:.0f} DRAM requests (x64 B, factor "
              f"{cal['dram_wr']:.5f}); FETCH_SIZE {copy['fetch'][1]['FETCH_SIZE']:.0f} KiB (factor "
              f"{cal['fetch']:.4f}), WRITE_SIZE {copy['write'][1]['WRITE_SIZE']:.0f} KiB (factor {cal['write']:.4f}).",
              "* The L2 sees requests leave for memory; whether the memory-side cache serves some of",
              "  them is not visible to these counters.", "",
              "| step | kernel | grid | trace avg ms | int8 GOP | bf16 TFLOP | MFMA busy | DRAM read GB | "
              "DRAM write GB | DRAM GB/s | FETCH+WRITE GB | L2 hit |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    lines += rows
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "prefill_flat_10m_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    a = kern.get("attention")
    with open(os.path.join(ROOT, "profiles", "attn_traffic.json"), "w") as f:
        json.dump({"workload": "flat_10m", "src_hash": src_hash(ATTN_SRC),
                   "bytes_per_launch": a["fetch_bytes"] + a["write_bytes"] if a else None,
                   "dram_bytes_per_launch": a["dram_read_bytes"] + a["dram_write_bytes"] if a else None,
                   "profile_avg_ms": a["trace_avg_ms"] if a else None,
                   "kernels": kern, "calibration": cal, "command": command}, f, indent=1)
    print("\n".join(lines))


def summarize_decode(args):
    """Decode kernel table from a rocprofv3 --stats CSV of `bench.py --profile-decode`."""
    import csv
    stats_csv, command = args.summarize_decode
    wl = S.WORKLOADS["decode_1m"]
    stats = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics: LSA decode, {wl.nseq} sequences x {wl.T} keys, "
             f"{wl.steps} steps (run twice)", "", f"Command: `{command}`", "",
             "Per-step kernels are called 2 x 256 = 512 times; the index build kernels run once "
             "per sequence before the steps.", "",
             "| kernel | calls | average us | total ms |", "|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        if "lsa" not in r["Name"]:
            continue
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['TotalDurationNs'])/1e6:.3f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "decode_1m_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_train(args):
    """Training-step kernel table from a rocprofv3 --stats CSV of `bench.py --train`."""
    import csv
    stats_csv, command = args.summarize_train
    wl = S.WORKLOADS["train_128k"]
    stats = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics: LSA training step of one layer, T={wl.T}, every "
             f"position a query (Hq={wl.Hq}, Hkv={wl.Hkv}, D={wl.D}, select "
             f"{wl.budget}+{wl.window}+{wl.sinks})", "", f"Command: `{command}`", "",
             "Each step: index build, select, grouped forward with log-sum-exp (sinks and "
             "window k_attn_swin, the plan: latent neighbours k_grp_nn, sort, unions "
             "k_grp_union; the walk k_attn_grp), backward (the plan again, dQ window pass "
             "k_bwd_dq<.., 1> and union walk k_bwd_dq_grp, then k_bwd_dkv band / long range / "
             "sinks and the list kernels); 4 steps (1 warmup + 3 timed).", "",
             "| kernel | calls | average ms | total ms |", "|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        if "lsa" not in r["Name"]:
            continue
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs'])/1e6:.3f} | "
                     f"{float(r['TotalDurationNs'])/1e6:.2f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "train_128k_rocprof.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="flat_10m", choices=["flat_10m", "flat_1m", "tree_10m", "tree3_10m"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-tree", action="store_true")
    ap.add_argument("--no-full", action="store_true",
                    help="skip the whole 10M prefill (320 chunks) of the default line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 1M and tiny Flat prefill steps of the default line")
    ap.add_argument("--profile", action="store_true",
                    help="one prefill step plus a 2 GiB calibration copy (for rocprofv3 runs)")
    ap.add_argument("--full-prefill", action="store_true",
                    help="the whole context chunk by chunk (index grown from empty); prints its own line")
    ap.add_argument("--train", action="store_true",
                    help="only the 128k training step (forward + backward of one layer)")
    ap.add_argument("--long-decode", action="store_true",
                    help="decode at 2M, 4M and 10M keys per sequence (indexes beyond the "
                         "register-resident select)")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only the decode benchmark (for rocprofv3 kernel traces)")
    ap.add_argument("--summarize-decode", nargs=2, metavar=("STATS", "COMMAND"),
                    help="write the decode kernel summary under profiles/ from a rocprofv3 stats CSV")
    ap.add_argument("--summarize-train", nargs=2, metavar=("STATS", "COMMAND"),
                    help="write the training-step kernel summary under profiles/ from a rocprofv3 stats CSV")
    ap.add_argument("--summarize-prefill", nargs=2, metavar=("DIR", "COMMAND"),
                    help="write the prefill summaries under profiles/ from the rocprofv3 outputs of "
                         "`bench.py --profile` (DIR/trace and one DIR/<pass> per counter pass)")
    args = ap.parse_args()
    if args.summarize_prefill:
        summarize_prefill(args)
        return
    if args.summarize_decode:
        summarize_decode(args)
        return
    if args.summarize_train:
        summarize_train(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the LSA hot path here is built and timed on a "
              "single MI355X (--gpus 1); multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)
    workers_pool = None
    if not (args.no_cpu or args.profile or args.profile_decode or args.full_prefill or args.train
            or args.long_decode):
        # forked before anything touches the GPU; the workers only run the CPU oracle
        import multiprocessing as mp
        workers_pool = mp.get_context("fork").Pool(min(16, os.cpu_count() or 1))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    L.lib()
    if args.profile:
        profile_run(args, dev)
        return
    if args.full_prefill:
        fp = bench_full_prefill(args, dev)
        print(json.dumps({"metric": "LSA layer whole-prefill time (all chunks, index grown chunk by chunk)",
                          "value": fp["total_s"], "unit": "s", "higher_is_better": False,
                          "n_gpus": 1, "data": "synthetic", "config": fp}), flush=True)
        return
    if args.train:
        tr = bench_train(args, dev)
        print(json.dumps({"metric": "LSA layer training step (fwd + bwd) tokens/s at 128k",
                          "value": tr["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                          "data": "synthetic", "config": tr}), flush=True)
        return
    if args.long_decode:
        import dataclasses
        runs = []
        for T, nseq in ((2 << 20, 4), (4 << 20, 4), (10 << 20, 2)):
            wl = dataclasses.replace(S.WORKLOADS["decode_1m"], name=f"decode_{T >> 20}m", T=T, nseq=nseq,
                                     steps=64)
            d = bench_decode(args, dev, wl)
            log(f"[bench] decode {T >> 20}M keys x {nseq}: {d['tokens_per_s']:.0f} tok/s "
                f"({d['ms_per_step']:.3f} ms/step, frac {d['roofline']['frac']:.2f})")
            runs.append(d)
            torch.cuda.empty_cache()
        # the same sequences on a two-level Tree index (G=64, S=64, R=32)
        tree_runs = []
        for T, nseq in ((2 << 20, 4), (10 << 20, 2)):
            wl = dataclasses.replace(S.WORKLOADS["decode_1m"], name=f"decode_tree_{T >> 20}m", T=T, nseq=nseq,
                                     steps=64, tree_group=64, tree_super=64, tree_iters=4, tree_top=32)
            d = bench_decode(args, dev, wl)
            log(f"[bench] Tree decode {T >> 20}M keys x {nseq}: {d['tokens_per_s']:.0f} tok/s "
                f"({d['ms_per_step']:.3f} ms/step)")
            tree_runs.append(d)
            torch.cuda.empty_cache()
        print(json.dumps({"metric": "LSA decode tokens/s at long contexts", "value": runs[-1]["tokens_per_s"],
                          "unit": "tokens/s", "higher_is_better": True, "n_gpus": 1, "data": "synthetic",
                          "config": {"workload": "decode at 2M / 4M / 10M keys per sequence (Flat; value: 10M), "
                                                 "and on a Tree index at 2M / 10M", "runs": runs,
                                     "tree_runs": tree_runs}}),
              flush=True)
        return
    if args.profile_decode:
        d = bench_decode(args, dev)
        log(f"[profile] decode {d['tokens_per_s']:.0f} tok/s ({d['ms_per_step']:.3f} ms/step)")
        return

    res = bench_prefill(args, dev)
    wl = res["wl"]
    log(f"[bench] prefill step {res['ms_per_step']:.2f} ms (append/select/attn "
        f"{res['phase_ms'][0]:.3f}/{res['phase_ms'][1]:.3f}/{res['phase_ms'][2]:.3f} ms), "
        f"walk {res['achieved_gbs']:.0f} GB/s per-query accounting, {res['union_gbs']:.0f} GB/s of union bytes")
    dense = None if args.no_dense else bench_dense(res, dev)
    if dense:
        log(f"[bench] dense scan {dense['ms_per_chunk']:.1f} ms for {dense['queries']} queries "
            f"(frac {dense['roofline']['frac']:.3f} of its int8 roof)")
    tree = None
    if not args.no_tree and wl.name == "flat_10m":
        tree = bench_tree_same_data(res, dev, args.steps, args.warmup)
        log(f"[bench] tree_10m step {tree['ms_per_step']:.2f} ms, selected keys per query "
            f"{tree['selected_keys_per_query']}")

    others = None
    if not args.no_configs and wl.name == "flat_10m":
        others = {}
        for name in ("flat_1m", "tiny_flat"):
            others[name] = bench_other_config(name, args, dev)
            log(f"[bench] {name} step {others[name]['ms_per_step']:.3f} ms "
                f"({others[name]['queries_per_s']:.0f} queries/s)")

    full = None
    if not args.no_full and wl.name == "flat_10m":
        full = bench_full_prefill(args, dev, data=(res["g"], res["latk"], res["K"], res["V"]))
        torch.cuda.empty_cache()

    # counters of the attention kernel (profiles/attn_traffic.json), valid
    # while the kernel's source is unchanged
    traffic = dram = prof_ms = None
    tf = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if os.path.exists(tf):
        with open(tf) as f:
            tj = json.load(f)
        if tj.get("src_hash") == src_hash(ATTN_SRC) and tj.get("workload") == wl.name:
            traffic = tj.get("bytes_per_launch")
            dram = tj.get("dram_bytes_per_launch")
            prof_ms = tj.get("profile_avg_ms")

    copy_gbs = measured_copy_gbs(dev)
    log(f"[bench] plain device copy {copy_gbs:.0f} GB/s (read + write)")

    decode = None
    if not args.no_decode:
        decode = bench_decode(args, dev)
        log(f"[bench] decode {decode['tokens_per_s']:.0f} tok/s ({decode['ms_per_step']:.3f} ms/step, "
            f"step roof {decode['roofline']['roof_ms'] * 1e3:.1f} us, frac {decode['roofline']['frac']:.2f})")

    train = None
    if not args.no_train:
        torch.cuda.empty_cache()
        train = bench_train(args, dev)

    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_baseline(res, workers_pool)
            log(f"[bench] cpu oracle {cpu['value']:.2f} queries/s, parity sample "
                f"{cpu['parity_sample']}")
        except Exception as e:  # report, never hide
            log(f"[bench] cpu baseline failed: {e!r}")
            cpu = {"value": None, "error": repr(e)}

    if workers_pool is not None:
        workers_pool.close()
        workers_pool.join()
    value = res["n"] / (res["ms_per_step"] / 1e3)
    roof_ms = layer_roof_ms(wl, res, res["attn_phase_bytes_per_query"])    # every query's rows
    roof_ms_grouped = layer_roof_ms(wl, res, res["attn_phase_bytes"])      # the unions
    line = {
        "metric": "LSA layer prefill queries/s at T=10M (32k chunk); decode tok/s; % roofline",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "context_tokens": wl.T, "chunk_queries": wl.chunk,
                   "index": f"Flat p={wl.pool} blocks={wl.block} buckets={wl.buckets} iters={wl.iters}"
                   + (f" tree G={wl.tree_group} S={wl.tree_super} R={wl.tree_top}" if wl.tree_group else "")
                   + (f" top G2={wl.tree2_group} S2={wl.tree2_super} R2={wl.tree2_top}"
                      if wl.tree2_group else ""),
                   "select": f"{wl.budget}+{wl.window}+{wl.sinks}",
                   "attention": f"GQA {wl.Hq}/{wl.Hkv} D={wl.D} bf16"},
        "roofline": {"kernel": f"{ATTN_KERNEL} (sparse GQA attention, grouped long-range walk)",
                     "bound": "hbm",
                     "achieved": res["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": res["achieved_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "accounting": "algorithmic bytes count every query's long-range K/V rows (reuse "
                                   "not credited); the walk reads each group's union of them once, so "
                                   "the rate passes the HBM peak; union_* fields are the bytes it reads",
                     "dram_bytes_per_launch": dram,
                     "algorithmic_bytes_per_launch": res["attn_bytes"],
                     "union_bytes_per_launch": res["attn_union_bytes"],
                     "union_achieved": res["union_gbs"], "union_frac": res["union_gbs"] / HBM_PEAK_GBS,
                     "avg_launch_ms": res["attn_ms"],
                     "profile_avg_launch_ms": prof_ms,
                     "frac_at_profile_avg": (res["attn_bytes"] / (prof_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
                                             if prof_ms else None),
                     "union_frac_at_profile_avg": (res["attn_union_bytes"] / (prof_ms * 1e-3) / 1e9
                                                   / HBM_PEAK_GBS if prof_ms else None),
                     "measured_copy_gbs": copy_gbs,
                     "layer": {"roof_ms": roof_ms, "measured_ms": res["ms_per_step"],
                               "frac": roof_ms / res["ms_per_step"],
                               "roof_ms_grouped_bytes": roof_ms_grouped,
                               "frac_grouped_bytes": roof_ms_grouped / res["ms_per_step"]}},
        "cpu_baseline": cpu,
        "phases_ms": {"append": res["phase_ms"][0], "select": res["phase_ms"][1],
                      "attention": res["phase_ms"][2]},
        "grouped_attention": res["grouped"],
        "step_event_ms": res["step_event_ms"],
        "fused_entry_point_identical": res["fused_same"],
        "select_roofline": {"roof_ms": select_roof_ms(wl, res["n"]), "measured_ms": res["phase_ms"][1],
                            "frac": select_roof_ms(wl, res["n"]) / res["phase_ms"][1]},
        "selected_keys_per_query": res["cnt_mean"],
        "index_build_keys_per_s": wl.T / (res["build_ms"] * 1e-3),
        "index_build": {"keys": wl.T, "ms": res["build_ms"], "roof_ms": build_roof_ms(wl),
                        "frac": build_roof_ms(wl) / res["build_ms"]},
        "tree_10m": tree,
        "other_configs": others,
        "full_prefill_10m": full,
        "decode": decode,
        "dense_scan": dense,
        "train_step_128k": train,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
