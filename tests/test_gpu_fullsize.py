"""GPU parity at the benchmarked sizes, in the benchmarked launch configuration.

Each test runs the path the benchmark times (index prebuilt over the context
before the chunk, then the fused prefill-chunk entry point; or 256 decode
steps) and checks, against the CPU oracle built block by block in worker
processes:
* every block's centroids and member lists bit-exactly;
* every selection row: the key count (min(t + 1, budget + window + sinks)),
  distinct keys, causality, window and sinks present, -1 padding, and the
  row equal to the GPU exact kernel's on the same index;
* the selected key sets of 1024 queries bit-exactly against the oracle
  (first, last and block-boundary queries included);
* the attention of 1024 queries within 2e-3 normwise (float32 output of the
  same kernel), with the bf16 output equal to its round-to-nearest-even;
* decode: every (sequence, step) query of the 256 steps, selection and
  attention.
The oracle's selections and attention outputs are computed in the worker
pool (oracle/parallel_refs.py).
"""
import numpy as np
import pytest
import torch

import lsa_synth as S
import oracle as O
from oracle.parallel_build import build_cache_parallel
from oracle.parallel_refs import decode_many, select_many

from test_gpu_parity import (TOL, check_index, normwise, oracle_attention, rne_bf16_bits)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _L():
    import hierarchical_sparse_attention_lsa_amd as L
    return L


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _oparams(wl):
    return O.IndexParams(wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group, wl.tree_super,
                         wl.tree_iters, wl.tree2_group, wl.tree2_super, wl.tree2_iters)


def _sample_positions(wl, n_sel, seed):
    n, t0 = wl.chunk, wl.T - wl.chunk
    kpb = wl.pool * wl.block
    fixed = sorted(set(i for i in [0, 1, n - 1, n - 2, kpb - 1, kpb, kpb + 1, n // 2 - 1, n // 2]
                       if 0 <= i < n))
    rng = np.random.default_rng(seed)
    others = np.setdiff1d(np.arange(n), fixed)
    rest = rng.choice(others, n_sel - len(fixed), replace=False).tolist()
    return sorted(fixed + rest)


def _gpu_prefill(wl, dev, out_f32_too=True, early=(0, 0)):
    """The benchmarked step: prebuilt index, then lsa_prefill_chunk (bf16 out);
    the same chunk again with a float32 output; and the exact selection
    kernel's rows for the chunk's queries on the same index."""
    L = _L()
    g = S.Synth(wl)
    n, t0 = wl.chunk, wl.T - wl.chunk
    latk = g.latk(0, wl.T, device=dev, chunk=1 << 22)
    K = torch.empty((wl.T, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0, chunk=1 << 18)
    g.fill_rows("v", V, 0, chunk=1 << 18)
    latq = g.latq_rows(torch.arange(t0, wl.T, device=dev), device=dev)
    q = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    g.fill_rows("q", q, t0)
    ix = L.LsaIndex(L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group,
                                  wl.tree_super, wl.tree_iters, wl.T, wl.tree2_group,
                                  wl.tree2_super, wl.tree2_iters), dev)
    ix.build(latk[:t0])
    snap = ix.snapshot()
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, *early, wl.tree2_top)
    idx = torch.empty((n, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((n,), dtype=torch.int32, device=dev)
    o16 = ix.prefill_chunk(latk[t0:], latq, q, K, V, sp, L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0),
                           idx=idx, cnt=cnt)
    o32 = None
    if out_f32_too:
        ix.restore(snap)
        o32 = ix.prefill_chunk(latk[t0:], latq, q, K, V, sp,
                               L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0))
    qpos = torch.arange(t0, wl.T, dtype=torch.int32, device=dev)
    idx_x, cnt_x = ix.select(latq, qpos, sp, use_workspace=False)
    torch.cuda.synchronize()
    res = dict(g=g, idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(), o16=o16, o32=o32,
               idx_exact=idx_x.cpu().numpy(), cnt_exact=cnt_x.cpu().numpy(),
               arrays={k: v.cpu() for k, v in ix.arrays().items()})
    del K, V, latk
    torch.cuda.empty_cache()
    return res


def oracle_attention_rows(g, wl, positions, sels, dev, label):
    """Float64 oracle attention of the query at positions[i] over the rows
    sels[i].  Q, K and V rows come from the workload's seeded generator run on
    the device (the counter-based generator gives the same bits on the host,
    checked here on the first query's rows), then the oracle runs on the host."""
    out = []
    for i, (t, sel) in enumerate(zip(positions, sels)):
        rows = torch.from_numpy(np.asarray(sel, dtype=np.int64)).to(dev)
        kb, vb = g.k_rows(rows, device=dev).cpu(), g.v_rows(rows, device=dev).cpu()
        qb = g.q_rows(torch.tensor([t], device=dev), device=dev).cpu()
        if i == 0:
            r8 = torch.from_numpy(np.asarray(sel[:8], dtype=np.int64))
            assert torch.equal(kb[:8].view(torch.int16), g.k_rows(r8).view(torch.int16))
            assert torch.equal(vb[:8].view(torch.int16), g.v_rows(r8).view(torch.int16))
            assert torch.equal(qb.view(torch.int16), g.q_rows(torch.tensor([t])).view(torch.int16))
        K = O.bf16_to_f64(kb.view(torch.int16).numpy())
        V = O.bf16_to_f64(vb.view(torch.int16).numpy())
        q = O.bf16_to_f64(qb.view(torch.int16).numpy())[0]
        out.append(O.attend(q, K, V, wl.Hkv))
        if (i + 1) % 256 == 0:
            print(f"  {label}: oracle attention {i + 1}/{len(positions)}", flush=True)
    return np.stack(out)


def check_rows(idx, cnt, positions, budgets, window, sinks):
    """Every selection row: count = min(t + 1, budget + window + sinks),
    distinct keys in [0, t], the window and the sinks present, -1 padding."""
    t = np.asarray(positions, dtype=np.int64)
    want = np.minimum(t + 1, np.asarray(budgets) + window + sinks)
    assert np.array_equal(cnt, want), f"{int((cnt != want).sum())} rows with a wrong key count"
    width = idx.shape[1]
    live = np.arange(width)[None, :] < cnt[:, None]
    assert (idx[~live] == -1).all(), "padding"
    big = np.iinfo(np.int32).max
    srt = np.sort(np.where(live, idx, big), axis=1)
    assert (srt[:, 0] >= 0).all()
    lv = np.arange(width)[None, :] < cnt[:, None]
    assert (np.diff(srt, axis=1)[lv[:, 1:]] > 0).all(), "repeated keys"
    last = np.take_along_axis(srt, (cnt - 1)[:, None].astype(np.int64), axis=1)[:, 0]
    assert (last <= t).all(), "a key past its query"
    in_win = (srt >= (t - window + 1)[:, None]) & (srt <= t[:, None])
    assert np.array_equal(in_win.sum(1), np.minimum(window, t + 1)), "window"
    assert np.array_equal((srt < sinks).sum(1), np.minimum(sinks, t + 1)), "sinks"


def _check_prefill(wl, res, ref, pool, n_sel, n_att, seed, early=(0, 0)):
    n, t0 = wl.chunk, wl.T - wl.chunk
    check_index(res["arrays"], ref)
    print(f"  {wl.name}: index bit-exact", flush=True)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, *early, wl.tree2_top)
    positions = np.arange(t0, wl.T)
    check_rows(res["idx"], res["cnt"], positions, [osp.budget_at(int(t)) for t in positions],
               wl.window, wl.sinks)
    assert np.array_equal(res["cnt"], res["cnt_exact"]) and np.array_equal(res["idx"], res["idx_exact"]), \
        f"{int((res['idx'] != res['idx_exact']).any(1).sum())} rows differ from the exact kernel's"
    print(f"  {wl.name}: all {n} rows valid and equal to the exact kernel's", flush=True)
    pos = _sample_positions(wl, n_sel, seed)
    latq = res["g"].latq_rows(torch.tensor([t0 + i for i in pos])).numpy()   # host-generated
    sels = select_many(pool, ref, latq, [t0 + i for i in pos], osp)
    for i, ref_sel in zip(pos, sels):
        got = np.sort(res["idx"][i, :res["cnt"][i]])
        assert np.array_equal(got, ref_sel), f"query at position {t0 + i}"
    print(f"  {wl.name}: {len(pos)} selections bit-exact", flush=True)
    att = pos[:: max(1, len(pos) // n_att)][:n_att]
    bysel = dict(zip(pos, sels))
    refo = oracle_attention_rows(res["g"], wl, [t0 + i for i in att], [bysel[i] for i in att],
                                 torch.device("cuda:0"), wl.name)
    o32 = res["o32"].cpu().numpy()[att].astype(np.float64)
    err = normwise(o32, refo)
    per_th = float((np.abs(o32 - refo).max(-1) / np.abs(refo).max(-1)).max())
    print(f"{wl.name}: {n} rows checked (count, causality, window, sinks; equal to the exact kernel), "
          f"{len(pos)} selections bit-exact, attention of {len(att)} queries: normwise error {err:.3e}, "
          f"worst (token, head) {per_th:.3e}")
    assert err <= TOL
    o16 = res["o16"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o16, rne_bf16_bits(res["o32"].cpu().numpy()))


@pytest.fixture(scope="module")
def oracle_1m(oracle_pool):
    wl = S.WORKLOADS["flat_1m"]
    cache, latk = build_cache_parallel(wl.name, wl.T, oracle_pool)
    return cache, latk


# (early_budget, early_until): the second keeps 2048 long-range keys for the
# first half of the chunk and the full budget from the middle on
@pytest.mark.parametrize("early", [(0, 0), (2048, (1 << 20) - (1 << 14))])
def test_flat_1m_prefill_chunk(oracle_1m, oracle_pool, early):
    dev = _dev()
    wl = S.WORKLOADS["flat_1m"]
    res = _gpu_prefill(wl, dev, early=early)
    cache, latk = oracle_1m
    ref = O.build_index(latk, wl.T, _oparams(wl), dict(cache))
    _check_prefill(wl, res, ref, oracle_pool, n_sel=1024, n_att=1024, seed=1 + early[0], early=early)


@pytest.fixture(scope="module")
def oracle_10m(oracle_pool):
    wl = S.WORKLOADS["flat_10m"]
    cache, latk = build_cache_parallel(wl.name, wl.T, oracle_pool)
    return cache, latk


def test_flat_10m_prefill_chunk(oracle_10m, oracle_pool):
    dev = _dev()
    wl = S.WORKLOADS["flat_10m"]
    res = _gpu_prefill(wl, dev)
    cache, latk = oracle_10m
    ref = O.build_index(latk, wl.T, _oparams(wl), dict(cache))
    _check_prefill(wl, res, ref, oracle_pool, n_sel=1024, n_att=1024, seed=2)


def test_tree_10m_prefill_chunk(oracle_10m, oracle_pool):
    dev = _dev()
    wl = S.WORKLOADS["tree_10m"]
    res = _gpu_prefill(wl, dev)
    cache, latk = oracle_10m
    ref = O.build_index(latk, wl.T, _oparams(wl), dict(cache))
    assert ref.n_grp == 10 and ref.sup_centroids.shape[0] == 640
    _check_prefill(wl, res, ref, oracle_pool, n_sel=1024, n_att=1024, seed=3)


def test_tree3_10m_prefill_chunk(oracle_10m, oracle_pool):
    dev = _dev()
    wl = S.WORKLOADS["tree3_10m"]
    res = _gpu_prefill(wl, dev)
    cache, latk = oracle_10m
    ref = O.build_index(latk, wl.T, _oparams(wl), dict(cache))
    assert ref.n_grp2 == 2 and ref.top_centroids.shape[0] == 64
    _check_prefill(wl, res, ref, oracle_pool, n_sel=256, n_att=256, seed=4)


def test_decode_1m_256_steps(oracle_pool):
    dev = _dev()
    L = _L()
    wl = S.WORKLOADS["decode_1m"]
    cap = wl.T + wl.steps
    gens = [S.Synth(wl, seq=i) for i in range(wl.nseq)]
    K = torch.empty((wl.nseq, cap, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    ixs, lats = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap, device=dev, chunk=1 << 22)
        lats.append(lk)
        g.fill_rows("k", K[i], 0, chunk=1 << 18)
        g.fill_rows("v", V[i], 0, chunk=1 << 18)
        ix = L.LsaIndex(L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap), dev)
        ix.build(lk[:wl.T])
        ixs.append(ix)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap32 = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    wsb = L.workspace_bytes(L.binding.OP_DECODE, ixs[0].params, sp, ap32, wl.nseq)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    got = []
    new_pos = torch.arange(wl.T, cap, device=dev)
    lq_all = torch.stack([gens[i].latq_rows(new_pos, device=dev) for i in range(wl.nseq)], 1)
    q_all = torch.stack([gens[i].q_rows(new_pos, device=dev) for i in range(wl.nseq)], 1)
    for s in range(wl.steps):
        t = wl.T + s
        lk_new = torch.stack([lats[i][t] for i in range(wl.nseq)]).contiguous()
        out = L.decode_step(ixs, lk_new, lq_all[s].contiguous(), q_all[s].contiguous(), K, V, cap,
                            sp, ap32, ws=ws)
        idx, cnt = L.decode_selection(ws, wl.nseq, sp)
        got.append((idx.clone(), cnt.clone(), out.clone()))
    torch.cuda.synchronize()
    got = [(a.cpu().numpy(), b.cpu().numpy(), c.cpu().numpy()) for a, b, c in got]
    final_arrays = {k: v.cpu() for k, v in ixs[0].arrays().items()}
    del K, V, lats
    torch.cuda.empty_cache()
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    # every step's rows: count, causality, window, sinks, padding
    for s in range(wl.steps):
        idx, cnt, _ = got[s]
        check_rows(idx, cnt, [wl.T + s] * wl.nseq, [wl.budget] * wl.nseq, wl.window, wl.sinks)
    caches, lat0 = [], None
    for i in range(wl.nseq):
        cache, lat_i = build_cache_parallel(wl.name, wl.T, oracle_pool, seq=i)   # host-generated
        caches.append(cache)
        print(f"  decode: sequence {i}: oracle blocks clustered", flush=True)
        if i == 0:
            lat0 = np.concatenate([lat_i, gens[0].latk(wl.T, cap).numpy()])
    print("  decode: oracle indexes built", flush=True)
    refs = decode_many(oracle_pool, wl.name, wl.T, wl.steps, _oparams(wl), osp, caches)
    worst, worst_th = 0.0, 0.0
    for i in range(wl.nseq):
        sels = refs[i]
        for s in range(wl.steps):
            idx, cnt, out = got[s]
            assert np.array_equal(np.sort(idx[i, :cnt[i]]), sels[s]), f"sequence {i} step {s}"
        print(f"  decode: sequence {i}: {wl.steps} selections bit-exact", flush=True)
        outs = oracle_attention_rows(gens[i], wl, [wl.T + s for s in range(wl.steps)], sels,
                                     torch.device("cuda:0"), f"decode sequence {i}")
        o = np.stack([got[s][2][i] for s in range(wl.steps)]).astype(np.float64)
        worst = max(worst, normwise(o, outs))
        worst_th = max(worst_th, float((np.abs(o - outs).max(-1) / np.abs(outs).max(-1)).max()))
    print(f"decode: selections bit-exact at all {wl.steps} steps x {wl.nseq} sequences, attention "
          f"normwise error {worst:.3e} (worst (token, head) {worst_th:.3e})")
    assert worst <= TOL
    # the last step's index equals the oracle's over all keys
    check_index(final_arrays, O.build_index(lat0, cap, _oparams(wl), caches[0]))


def test_tree_decode_2m_four_sequences(oracle_pool):
    """Tree decode at 4 sequences x 2M keys (G=64, S=64, R=32): the 32 chosen
    supers of 128 carry about 5000 leaves, more than the Tree kernel's
    candidate list, so the streaming pair serves these sequences."""
    import dataclasses
    dev = _dev()
    L = _L()
    # same latents as decode_1m (the data depends on the workload's data id only)
    wl = dataclasses.replace(S.WORKLOADS["decode_1m"], name="decode_tree_2m", T=2 << 20, nseq=4,
                             steps=4, tree_group=64, tree_super=64, tree_iters=4, tree_top=32)
    cap = wl.T + wl.steps
    gens = [S.Synth(wl, seq=i) for i in range(wl.nseq)]
    K = torch.empty((wl.nseq, cap, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group, wl.tree_super,
                       wl.tree_iters, cap)
    ixs, lats = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap, device=dev, chunk=1 << 22)
        lats.append(lk)
        g.fill_rows("k", K[i], 0, chunk=1 << 18)
        g.fill_rows("v", V[i], 0, chunk=1 << 18)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:wl.T])
        ixs.append(ix)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    ap32 = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap32, wl.nseq), dtype=torch.uint8,
                     device=dev)
    check_steps = {0, wl.steps - 1}
    got = {}
    for s in range(wl.steps):
        t = wl.T + s
        pos = torch.tensor([t], device=dev)
        lk_new = torch.stack([lats[i][t] for i in range(wl.nseq)]).contiguous()
        lq = torch.cat([gens[i].latq_rows(pos, device=dev) for i in range(wl.nseq)]).contiguous()
        q = torch.cat([gens[i].q_rows(pos, device=dev) for i in range(wl.nseq)]).contiguous()
        out = L.decode_step(ixs, lk_new, lq, q, K, V, cap, sp, ap32, ws=ws)
        if s in check_steps:
            idx, cnt = L.decode_selection(ws, wl.nseq, sp)
            got[s] = (idx.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy())
    torch.cuda.synchronize()
    del K, V, lats
    torch.cuda.empty_cache()
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    worst = 0.0
    lat_h = []
    for i in range(wl.nseq):
        cache, lat0 = build_cache_parallel("decode_1m", wl.T, oracle_pool, seq=i)   # host-generated
        lat_h.append(np.concatenate([lat0, gens[i].latk(wl.T, cap).numpy()]))
        for s in sorted(check_steps):
            t = wl.T + s
            ref = O.build_index(lat_h[i], t + 1, _oparams(wl), cache)
            lq = gens[i].latq_rows(torch.tensor([t])).numpy()[0]
            sel = O.select(ref, lq, t, osp)
            idx, cnt, out = got[s]
            assert np.array_equal(np.sort(idx[i, :cnt[i]]), sel), f"sequence {i} step {s}"
            ro = oracle_attention(gens[i], wl, [t], [sel])[0]
            worst = max(worst, normwise(out[i].astype(np.float64), ro))
    print(f"tree decode 2M: selections bit-exact at {len(check_steps)} steps x {wl.nseq} sequences, "
          f"attention normwise error {worst:.3e}")
    assert worst <= TOL


def test_flat_1m_chunked_prefill_from_empty(oracle_1m):
    """The whole 1M context through lsa_prefill_chunk, 32 chunks from an empty
    index: the final index equals the oracle's build, and sampled queries of
    several chunks select the oracle's key sets and attend within tolerance."""
    dev = _dev()
    L = _L()
    wl = S.WORKLOADS["flat_1m"]
    n = wl.chunk
    nchunks = wl.T // n
    g = S.Synth(wl)
    latk = g.latk(0, wl.T, device=dev, chunk=1 << 22)
    K = torch.empty((wl.T, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0, chunk=1 << 18)
    g.fill_rows("v", V, 0, chunk=1 << 18)
    ix = L.LsaIndex(L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, wl.T), dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    q = torch.empty((n, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((n, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((n,), dtype=torch.int32, device=dev)
    checked = {0: [0, 1, 511, 512, 4095, 20000, n - 1], 1: [0, 7, 30000],
               15: [0, 12345, n - 1], nchunks - 1: [0, 9999, n - 2, n - 1]}
    got = {}
    for c in range(nchunks):
        t0 = c * n
        latq = g.latq_rows(torch.arange(t0, t0 + n, device=dev), device=dev)
        g.fill_rows("q", q, t0)
        out = ix.prefill_chunk(latk[t0:t0 + n], latq, q, K, V, sp, ap, idx=idx, cnt=cnt)
        if c in checked:
            rows = checked[c]
            got[c] = (idx[rows].cpu().numpy(), cnt[rows].cpu().numpy(), out[rows].cpu().numpy())
    torch.cuda.synchronize()
    arrays = {k: v.cpu() for k, v in ix.arrays().items()}
    del K, V
    torch.cuda.empty_cache()
    cache, latk_h = oracle_1m                                            # host-generated
    check_index(arrays, O.build_index(latk_h, wl.T, _oparams(wl), dict(cache)))
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    worst = 0.0
    for c, rows in checked.items():
        ref = O.build_index(latk_h, (c + 1) * n, _oparams(wl), dict(cache))
        pos = [c * n + r for r in rows]
        lq = g.latq_rows(torch.tensor(pos)).numpy()
        sels = [O.select(ref, lq[j], t, osp) for j, t in enumerate(pos)]
        gi, gc, go = got[c]
        for j, t in enumerate(pos):
            assert np.array_equal(np.sort(gi[j, :gc[j]]), sels[j]), f"chunk {c} position {t}"
        refo = oracle_attention(g, wl, pos, sels)
        worst = max(worst, normwise(go.astype(np.float64), refo))
    print(f"chunked prefill from empty: {sum(len(r) for r in checked.values())} selections bit-exact, "
          f"attention normwise error {worst:.3e}")
    assert worst <= TOL


def test_train_128k_backward(oracle_pool):
    """The benchmarked training step at 128k (every position a query, bf16
    forward output): dQ of sampled queries and dK / dV of the last keys
    (reached only through windows) against the oracle over its own
    selections, and the zero-sum / value-sum properties over all keys."""
    dev = _dev()
    L = _L()
    wl = S.WORKLOADS["train_128k"]
    T = wl.T
    g = S.Synth(wl)
    latk = g.latk(0, T, device=dev)
    K = torch.empty((T, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    q = torch.empty((T, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    do = torch.empty_like(q)
    for name, tt in (("k", K), ("v", V), ("q", q), ("do", do)):
        g.fill_rows(name, tt, 0)
    ix = L.LsaIndex(L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, T), dev)
    ix.build(latk)
    pos = torch.arange(T, device=dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    latq = g.latq_rows(pos, device=dev)
    idx, cnt = ix.select(latq, pos.to(torch.int32), sp)
    # properties over all keys, with a float32 forward output (exact row sums):
    # the softmax gradients sum to zero over the keys; the value gradients sum
    # to the upstream gradients of each KV head's query heads
    ap32 = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    lse32 = torch.empty((T, wl.Hq), dtype=torch.float32, device=dev)
    out32 = L.sparse_attn_grouped(q, K, V, idx, cnt, 0, sp, ap32, lse=lse32)    # the benchmarked forward
    _, dk32, dv32 = L.sparse_attn_bwd(ix, q, K, V, idx, cnt, 0, sp, ap32, out32, lse32, do)
    G = wl.Hq // wl.Hkv
    dks = dk32.double().sum(0)
    assert float(dks.abs().max()) <= 1e-4 * float(dk32.double().abs().sum(0).max())
    want = do.double().view(T, wl.Hkv, G, wl.D).sum((0, 2))
    assert float((dv32.double().sum(0) - want).abs().max()) <= 1e-4 * float(want.abs().max())
    del out32, lse32, dk32, dv32
    # the benchmarked configuration: grouped forward, bf16 output, groups by
    # the query latents
    lse = torch.empty((T, wl.Hq), dtype=torch.float32, device=dev)
    out = L.sparse_attn_grouped(q, K, V, idx, cnt, 0, sp, ap, lse=lse, latq=latq)
    dq, dk, dv = L.sparse_attn_bwd(ix, q, K, V, idx, cnt, 0, sp, ap, out, lse, do, latq=latq)
    torch.cuda.synchronize()
    # oracle over its own selections
    cache, latk_h = build_cache_parallel(wl.name, T, oracle_pool)
    ref = O.build_index(latk_h, T, _oparams(wl), cache)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)

    def f64(t):
        return O.bf16_to_f64(t.view(torch.int16).numpy())

    def grads(t):
        sel = O.select(ref, g.latq_rows(torch.tensor([t])).numpy()[0], t, osp)
        rows = torch.from_numpy(sel)
        Kr, Vr = f64(g.k_rows(rows)), f64(g.v_rows(rows))
        qt = f64(g.q_rows(torch.tensor([t])))[0]
        dot = f64(g.do_rows(torch.tensor([t])))[0]
        o = O.round_bf16(O.attend(qt, Kr, Vr, wl.Hkv))        # the stored bf16 output
        return sel, O.attend_backward(qt, Kr, Vr, dot, wl.Hkv, o=o)

    qs = [0, 1, 511, 512, 513, 4100, 20000, 77777, T - 300, T - 1]
    got = dq[qs].cpu().numpy().astype(np.float64)
    refq = np.stack([grads(t)[1][0] for t in qs])
    eq = normwise(got, refq)
    # keys after T - window reach no long-range row: their gradients come from the
    # windows of the queries t = j .. T-1
    keys = [T - 1, T - 2, T - 57, T - 200]
    j0 = min(keys)
    dK = {j: np.zeros((wl.Hkv, wl.D)) for j in keys}
    dV = {j: np.zeros((wl.Hkv, wl.D)) for j in keys}
    for t in range(j0, T):
        sel, (_, gk, gv) = grads(t)
        for j in keys:
            if j <= t:
                r = int(np.searchsorted(sel, j))
                assert sel[r] == j
                dK[j] += gk[r]
                dV[j] += gv[r]
    ek = normwise(dk[keys].cpu().numpy().astype(np.float64), np.stack([dK[j] for j in keys]))
    ev = normwise(dv[keys].cpu().numpy().astype(np.float64), np.stack([dV[j] for j in keys]))
    print(f"train 128k: dQ ({len(qs)} queries) {eq:.2e}, dK {ek:.2e}, dV {ev:.2e} normwise")
    assert max(eq, ek, ev) <= TOL
