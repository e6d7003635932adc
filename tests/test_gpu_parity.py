"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Index arrays and selected key sets must match bit-exactly; attention must
match the float64 oracle within 2e-3 normwise relative error
(max |gpu - ref| / max |ref| over the compared tensor), measured on the
kernel's float32 output, and the bf16 output must be the round-to-nearest-
even of that float32 output.
"""
import dataclasses

import numpy as np
import pytest
import torch

import lsa_synth as S
import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _L():
    import hierarchical_sparse_attention_lsa_amd as L
    return L


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _iparams(wl, max_tokens=None):
    L = _L()
    return L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group,
                         wl.tree_super, wl.tree_iters, max_tokens or wl.T, wl.tree2_group,
                         wl.tree2_super, wl.tree2_iters)


def _oparams(wl):
    return O.IndexParams(wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group, wl.tree_super,
                         wl.tree_iters, wl.tree2_group, wl.tree2_super, wl.tree2_iters)


def check_index(gpu_arrays, ref: O.Index, blocks=None):
    """Bit-exact comparison of the GPU index with the oracle's (optionally a subset of blocks)."""
    a = {k: v.cpu().numpy() for k, v in gpu_arrays.items()}
    assert a["cent"].shape[0] == ref.n_bkt
    assert np.array_equal(a["pooled"], ref.pooled), "pooled vectors"
    counts = np.array([len(m) for m in ref.members], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)[:-1]]) if len(counts) else counts
    mem = np.concatenate(ref.members) if ref.members else np.zeros(0, np.int64)
    if blocks is None:
        assert np.array_equal(a["cent"], ref.centroids), "centroids"
        assert np.array_equal(a["bcnt"], counts), "bucket counts"
        assert np.array_equal(a["boff"], offs), "bucket offsets"
        assert np.array_equal(a["bmem"], mem), "members"
    else:
        C, N = ref.params.buckets, ref.params.block
        for b in blocks:
            sl = slice(b * C, (b + 1) * C)
            assert np.array_equal(a["cent"][sl], ref.centroids[sl]), f"centroids block {b}"
            assert np.array_equal(a["bcnt"][sl], counts[sl]), f"counts block {b}"
            assert np.array_equal(a["boff"][sl], offs[sl]), f"offsets block {b}"
            assert np.array_equal(a["bmem"][b * N:(b + 1) * N], mem[b * N:(b + 1) * N])
    nz = counts > 0
    first = np.array([m[0] if len(m) else 2 ** 31 - 1 for m in ref.members])
    last = np.array([m[-1] if len(m) else -1 for m in ref.members])
    if blocks is None:
        assert np.array_equal(a["bfirst"], first) and np.array_equal(a["blast"], last)
    if ref.sup_centroids is not None and blocks is None:
        assert np.array_equal(a["scent"], ref.sup_centroids), "super centroids"
        sc = np.array([len(m) for m in ref.sup_members])
        assert np.array_equal(a["scnt"], sc)
        smem = np.concatenate(ref.sup_members) if ref.sup_members else np.zeros(0)
        assert np.array_equal(a["smem"], smem)
    if ref.top_centroids is not None and blocks is None:
        assert np.array_equal(a["tcent"], ref.top_centroids), "top-node centroids"
        tcn = np.array([len(m) for m in ref.top_members])
        assert np.array_equal(a["tcnt"], tcn)
        toff = np.concatenate([[0], np.cumsum(tcn)[:-1]]) if len(tcn) else tcn
        assert np.array_equal(a["toff"], toff)
        tmem = np.concatenate(ref.top_members) if ref.top_members else np.zeros(0)
        assert np.array_equal(a["tmem"], tmem)


def check_selection(idx, cnt, refs, max_sel):
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    for i, ref in enumerate(refs):
        n = int(cnt[i])
        got = idx[i, :n]
        assert np.array_equal(np.sort(got), ref), f"query {i}: {n} vs {len(ref)} keys"
        assert (idx[i, n:] == -1).all()
        assert n <= max_sel


def oracle_attention(g: S.Synth, wl, positions, sels, scale=None):
    out = []
    for t, sel in zip(positions, sels):
        rows = torch.from_numpy(np.asarray(sel, dtype=np.int64))
        K = O.bf16_to_f64(g.k_rows(rows).view(torch.int16).numpy())
        V = O.bf16_to_f64(g.v_rows(rows).view(torch.int16).numpy())
        q = O.bf16_to_f64(g.q_rows(torch.tensor([t])).view(torch.int16).numpy())[0]
        out.append(O.attend(q, K, V, wl.Hkv, scale))
    return np.stack(out)


def normwise(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny():
    dev = _dev()
    wl = S.WORKLOADS["tiny_flat"]
    g = S.Synth(wl)
    latk = g.latk(0, wl.T)
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    return wl, g, latk, ref, dev


def test_tiny_index_bit_exact(tiny):
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)


def test_tiny_selection_bit_exact(tiny):
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    # the chunk's queries plus early positions (window-only, sinks overlap) and a ragged count
    pos = list(range(wl.T - wl.chunk, wl.T)) + [0, 1, 3, 4, 100, 127, 128, 131, 132, 133, 5000]
    lq = g.latq_rows(torch.tensor(pos))
    idx, cnt = ix.select(lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp)
    refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, refs, sp.max_sel)
    # determinism: a second run is bitwise identical (order included)
    idx2, cnt2 = ix.select(lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    # the exact refinement path alone (no workspace) gives the same rows
    idx3, cnt3 = ix.select(lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp,
                           use_workspace=False)
    assert torch.equal(idx, idx3) and torch.equal(cnt, cnt3)
    # the enqueued work ran without a device-side error
    L.check()


def test_select_every_position_as_a_query(tiny):
    """A training-like batch: every position of the tiny context is a query over
    the full index (most of the index lies past the early queries).  The list
    path (causal scan) matches the exact kernel on all rows and the oracle on
    a sample that includes the early positions."""
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    pos = torch.arange(wl.T, dtype=torch.int32)
    lq = g.latq_rows(pos.to(torch.int64))
    idx, cnt = ix.select(lq.to(dev), pos.to(dev), sp)
    idx_x, cnt_x = ix.select(lq.to(dev), pos.to(dev), sp, use_workspace=False)
    assert torch.equal(idx, idx_x) and torch.equal(cnt, cnt_x)
    rng = np.random.default_rng(7)
    sample = sorted(set(range(0, 1400, 7)) | set(rng.choice(wl.T, 300, replace=False).tolist()))
    refs = [O.select(ref, lq[t].numpy(), t, osp) for t in sample]
    check_selection(idx[sample], cnt[sample], refs, sp.max_sel)


def test_tiny_attention_within_tolerance(tiny):
    wl, g, latk, ref, dev = tiny
    L = _L()
    pos = list(range(wl.T - wl.chunk, wl.T))
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    lq = g.latq_rows(torch.tensor(pos))
    sels = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    max_sel = wl.max_sel
    idx = torch.full((len(pos), max_sel), -1, dtype=torch.int32)
    cnt = torch.zeros(len(pos), dtype=torch.int32)
    for i, s in enumerate(sels):
        idx[i, :len(s)] = torch.from_numpy(s[::-1].copy().astype(np.int32))   # any order
        cnt[i] = len(s)
    q = g.q_rows(torch.tensor(pos))
    K = torch.empty((wl.T, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    args = [t.to(dev) for t in (q, K, V, idx, cnt)]
    o32 = L.sparse_attn(*args, L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0))
    o16 = L.sparse_attn(*args, L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0))
    refo = oracle_attention(g, wl, pos, sels)
    err = normwise(o32.cpu().numpy().astype(np.float64), refo)
    print(f"tiny attention normwise error {err:.3e}")
    assert err <= TOL
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16),
                          rne_bf16_bits(o32.cpu().numpy()))


def test_tiny_prefill_chunk_fused(tiny):
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl), dev)
    t0 = wl.T - wl.chunk
    ix.build(latk[:t0].to(dev))
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    K = torch.empty((wl.T, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    pos = list(range(t0, wl.T))
    lq = g.latq_rows(torch.tensor(pos))
    q = g.q_rows(torch.tensor(pos))
    idx = torch.empty((wl.chunk, wl.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((wl.chunk,), dtype=torch.int32, device=dev)
    out = ix.prefill_chunk(latk[t0:].to(dev), lq.to(dev), q.to(dev), K.to(dev), V.to(dev), sp, ap,
                           idx=idx, cnt=cnt)
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    sels = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, sels, wl.max_sel)
    err = normwise(out.cpu().numpy().astype(np.float64), oracle_attention(g, wl, pos, sels))
    assert err <= TOL


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 4), (6, 2)])
def test_prefill_chunk_grouped_and_window_paths(tiny, Hq, Hkv):
    """lsa_prefill_chunk takes the grouped attention for G = Hq/Hkv in {4, 8,
    16} and the window kernel otherwise (G = 1, 3 here); both against the
    oracle on the same selections."""
    wl, g, latk, ref, dev = tiny
    L = _L()
    wl2 = dataclasses.replace(wl, Hq=Hq, Hkv=Hkv)
    g2 = S.Synth(wl2)
    t0 = wl.T - wl.chunk
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(Hq, Hkv, wl.D, 1, 0.0)
    K = torch.empty((wl.T, Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g2.fill_rows("k", K, 0)
    g2.fill_rows("v", V, 0)
    pos = list(range(t0, wl.T))
    lq = g.latq_rows(torch.tensor(pos))
    q = g2.q_rows(torch.tensor(pos))
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk[:t0].to(dev))
    idx = torch.empty((wl.chunk, sp.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((wl.chunk,), dtype=torch.int32, device=dev)
    out = ix.prefill_chunk(latk[t0:].to(dev), lq.to(dev), q.to(dev), K.to(dev), V.to(dev), sp, ap,
                           idx=idx, cnt=cnt)
    torch.cuda.synchronize()
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    sels = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, sels, wl.max_sel)
    err = normwise(out.cpu().numpy().astype(np.float64), oracle_attention(g2, wl2, pos, sels))
    print(f"prefill chunk G={Hq // Hkv}: normwise error {err:.3e}")
    assert err <= TOL


def test_position_dependent_budget(tiny):
    """Queries before early_until take early_budget long-range keys, later ones
    the full budget; the switch falls inside one launch.  Checked on the
    scan + resolve path, the exact path, the fused prefill chunk and the
    dense (every-key) selection."""
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    t0 = wl.T - wl.chunk
    pos = list(range(t0, wl.T)) + [0, 3, 131, 132, 5000, 9000]
    lq = g.latq_rows(torch.tensor(pos))
    pos_d = torch.tensor(pos, dtype=torch.int32, device=dev)
    for eb, eu in ((300, t0 + 37), (0, t0 + 64), (wl.budget, wl.T), (17, 6000), (200, 0)):
        sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0, eb, eu)
        osp = O.SelectParams(wl.budget, wl.window, wl.sinks, 0, eb, eu)
        refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
        idx, cnt = ix.select(lq.to(dev), pos_d, sp)
        check_selection(idx, cnt, refs, sp.max_sel)
        idx2, cnt2 = ix.select(lq.to(dev), pos_d, sp, use_workspace=False)
        assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    # fused prefill chunk with the switch in the middle of the chunk
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0, 400, t0 + 50)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, 0, 400, t0 + 50)
    ix2 = L.LsaIndex(_iparams(wl), dev)
    ix2.build(latk[:t0].to(dev))
    K = torch.empty((wl.T, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    cpos = list(range(t0, wl.T))
    clq = g.latq_rows(torch.tensor(cpos))
    q = g.q_rows(torch.tensor(cpos))
    idx = torch.empty((wl.chunk, wl.max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((wl.chunk,), dtype=torch.int32, device=dev)
    out = ix2.prefill_chunk(latk[t0:].to(dev), clq.to(dev), q.to(dev), K.to(dev), V.to(dev), sp,
                            L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0), idx=idx, cnt=cnt)
    torch.cuda.synchronize()
    sels = [O.select(ref, clq[i].numpy(), t, osp) for i, t in enumerate(cpos)]
    check_selection(idx, cnt, sels, wl.max_sel)
    assert len(sels[0]) < len(sels[-1])
    err = normwise(out.cpu().numpy().astype(np.float64), oracle_attention(g, wl, cpos, sels))
    assert err <= TOL
    # dense selection
    dpos = [5, 200, 1000, 2047, 4096, 5999, 3333]
    dlq = g.latq_rows(torch.tensor(dpos))
    sp = L.SelectParams(300, 128, 4, 0, 90, 3000)
    osp = O.SelectParams(300, 128, 4, 0, 90, 3000)
    idx, cnt = L.dense_select(latk[:6000].to(dev), dlq.to(dev),
                              torch.tensor(dpos, dtype=torch.int32, device=dev), sp)
    refs = [O.dense_select(latk[:6000].numpy(), dlq[i].numpy(), t, osp) for i, t in enumerate(dpos)]
    check_selection(idx, cnt, refs, sp.max_sel)


WINDOW_CASES = [
    # Hq, Hkv, D, qpos0, nq, budget, window, sinks
    (4, 1, 64, 0, 37, 120, 40, 5),        # G=4: 4 queries a wave; windows cut at 0, no long-range keys
    (8, 8, 128, 3000, 45, 200, 40, 5),    # G=1: 16 queries a wave, ragged group
    (16, 2, 64, 2040, 33, 200, 64, 3),    # G=8: 2 queries a wave
    (6, 2, 64, 100, 23, 80, 48, 7),       # G=3: 5 queries a wave, one column unused
    (16, 1, 128, 4000, 20, 150, 40, 5),   # G=16: one query a wave
    (4, 1, 64, 7, 50, 60, 4, 0),          # window = pool, no sinks
]


@pytest.mark.parametrize("case", WINDOW_CASES)
def test_window_attention_matches_oracle(case):
    """lsa_sparse_attn_window on rows laid out as the select writes them
    (long-range keys in shuffled order, then sinks, then window), built on
    the host from the oracle's selections."""
    dev = _dev()
    L = _L()
    Hq, Hkv, D, qpos0, nq, budget, window, sinks = case
    wl = S.Workload("win", 90, T=4096, ncomp=16, block=64, buckets=16, iters=2, chunk=0,
                    budget=budget, window=window, sinks=sinks, Hq=Hq, Hkv=Hkv, D=D)
    g = S.Synth(wl, data_cfg=90)
    latk = g.latk(0, wl.T)
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    pos = list(range(qpos0, qpos0 + nq))
    lq = g.latq_rows(torch.tensor(pos))
    osp = O.SelectParams(budget, window, sinks)
    sels = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    rng = np.random.default_rng(qpos0 + nq)
    idx = torch.full((nq, wl.max_sel), -1, dtype=torch.int32)
    cnt = torch.zeros(nq, dtype=torch.int32)
    for i, (t, sel) in enumerate(zip(pos, sels)):
        ws = max(0, t - window + 1)
        ns = max(0, min(sinks, ws))
        fixed = list(range(ns)) + list(range(ws, t + 1))
        assert set(fixed) <= set(sel.tolist())
        lr = np.array(sorted(set(sel.tolist()) - set(fixed)), dtype=np.int64)
        rng.shuffle(lr)
        row = np.concatenate([lr, np.array(fixed, dtype=np.int64)]).astype(np.int32)
        idx[i, :len(row)] = torch.from_numpy(row)
        cnt[i] = len(row)
    q = g.q_rows(torch.tensor(pos))
    K = torch.empty((wl.T, Hkv, D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    qd, Kd, Vd, idd, cd = (t.to(dev) for t in (q, K, V, idx, cnt))
    sp = L.SelectParams(budget, window, sinks, 0)
    o32 = L.sparse_attn_window(qd, Kd, Vd, idd, cd, qpos0, sp, L.AttnParams(Hq, Hkv, D, 1, 0.0))
    o16 = L.sparse_attn_window(qd, Kd, Vd, idd, cd, qpos0, sp, L.AttnParams(Hq, Hkv, D, 0, 0.0))
    g32 = L.sparse_attn(qd, Kd, Vd, idd, cd, L.AttnParams(Hq, Hkv, D, 1, 0.0))
    refo = oracle_attention(g, wl, pos, sels)
    err = normwise(o32.cpu().numpy().astype(np.float64), refo)
    err_generic = normwise(g32.cpu().numpy().astype(np.float64), refo)
    print(f"window attention {case}: normwise error {err:.3e} (generic kernel {err_generic:.3e})")
    assert err <= TOL and err_generic <= TOL
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16),
                          rne_bf16_bits(o32.cpu().numpy()))
    if Hq // Hkv in (4, 8, 16):
        # grouped: the same rows, long-range keys read once per group of queries
        gr32 = L.sparse_attn_grouped(qd, Kd, Vd, idd, cd, qpos0, sp, L.AttnParams(Hq, Hkv, D, 1, 0.0))
        gr16 = L.sparse_attn_grouped(qd, Kd, Vd, idd, cd, qpos0, sp, L.AttnParams(Hq, Hkv, D, 0, 0.0))
        err_g = normwise(gr32.cpu().numpy().astype(np.float64), refo)
        print(f"  grouped kernel {err_g:.3e}")
        assert err_g <= TOL
        assert np.array_equal(gr16.view(torch.int16).cpu().numpy().view(np.uint16),
                              rne_bf16_bits(gr32.cpu().numpy()))


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (8, 1, 128), (32, 2, 64)])
def test_grouped_attention_on_select_rows(tiny, Hq, Hkv, D):
    """lsa_sparse_attn_grouped on rows the Flat list path wrote (best bucket
    first, so neighbouring queries in the sorted order share most keys), for
    5000 queries (several sort tiles and merge passes, a ragged last group):
    every output against the window kernel's, sampled queries against the
    oracle on the oracle's own selections.  Then with the per-query union cap
    (the select budget) below some rows' long-range counts: those groups are
    walked row by row."""
    wl, g, latk, ref, dev = tiny
    L = _L()
    wl = dataclasses.replace(wl, Hq=Hq, Hkv=Hkv, D=D)
    g = S.Synth(wl)
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    qpos0, nq = 11000, 5000
    pos = torch.arange(qpos0, qpos0 + nq)
    lq = g.latq_rows(pos)
    eb, eu = 300, qpos0 + 1700          # the first 1700 queries take 300 long-range keys
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0, eb, eu)
    idx, cnt = ix.select(lq.to(dev), pos.to(torch.int32).to(dev), sp)
    q = g.q_rows(pos).to(dev)
    K = torch.empty((wl.T, Hkv, D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    K, V = K.to(dev), V.to(dev)
    ap32 = L.AttnParams(Hq, Hkv, D, 1, 0.0)
    win = L.sparse_attn_window(q, K, V, idx, cnt, qpos0, sp, ap32)
    grp = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32)
    gr16 = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, L.AttnParams(Hq, Hkv, D, 0, 0.0))
    # a cap of 300: the later queries' 1024-key rows go row by row
    sp_cap = L.SelectParams(eb, wl.window, wl.sinks, 0)
    cap = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp_cap, ap32)
    torch.cuda.synchronize()
    w = win.cpu().numpy().astype(np.float64)
    for name, o in (("grouped", grp), ("grouped, capped unions", cap)):
        e = normwise(o.cpu().numpy().astype(np.float64), w)
        print(f"{name} vs window kernel, {nq} queries: {e:.3e}")
        assert e <= TOL
    assert np.array_equal(gr16.view(torch.int16).cpu().numpy().view(np.uint16),
                          rne_bf16_bits(grp.cpu().numpy()))
    # the two halves in turn give the same bits, and so does a second call
    ws = torch.empty(L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap32, nq), dtype=torch.uint8,
                     device=dev)
    L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32, ws=ws, part="prepare")
    halves = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32, ws=ws, part="walk")
    again = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32)
    assert torch.equal(halves, grp) and torch.equal(again, grp)
    rng = np.random.default_rng(7)
    samp = sorted(set([0, 1, 1699, 1700, nq - 1] + rng.choice(nq, 40, replace=False).tolist()))
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, 0, eb, eu)
    sels = [O.select(ref, lq[i].numpy(), qpos0 + i, osp) for i in samp]
    check_selection(idx[samp], cnt[samp], sels, sp.max_sel)
    refo = oracle_attention(g, wl, [qpos0 + i for i in samp], sels)
    for name, o in (("grouped", grp), ("grouped, capped unions", cap)):
        e = normwise(o.cpu().numpy()[samp].astype(np.float64), refo)
        print(f"{name} vs oracle, {len(samp)} queries: {e:.3e}")
        assert e <= TOL


def _al256(x):
    return (x + 255) // 256 * 256


def _grouped_plan_from_ws(ws, nq, qpw, budget):
    """The query order (slot -> query) and the union sizes that
    lsa_attn_grouped_prepare leaves at the start of its workspace: the two
    sort-key buffers (8 bytes x the sort's padded size, the next power of two
    from 2048), the order, the union rows and masks (budget x qpw rounded up
    to 4 per group), then the union counts."""
    n_pad = 2048
    while n_pad < nq:
        n_pad *= 2
    ngrp = (nq + qpw - 1) // qpw
    ucap = (qpw * budget + 3) & ~3
    o_perm = 2 * _al256(n_pad * 8)
    o_ucnt = o_perm + _al256(nq * 4) + _al256(ngrp * ucap * 4) + _al256(ngrp * ucap)
    h = ws.cpu().numpy()
    perm = h[o_perm:o_perm + nq * 4].view(np.int32)
    ucnt = h[o_ucnt:o_ucnt + ngrp * 4].view(np.int32)
    return perm, ucnt


def _latent_order(latq, first, block=32768):
    """Host statement of the latent order: within each block of `block`
    consecutive queries, each query's nearest other query by squared distance
    (the j != i maximising 2 x_i.x_j - |x_j|^2, lowest j on ties; a lone
    query is its own), pointer jumping to the mutual pair each chain ends in,
    the pair's lower index as root; sorted by (first[root] >> 4, root, q)."""
    x = torch.from_numpy(latq.astype(np.float32))     # every partial sum an integer below 2^24: exact
    n = x.shape[0]
    nrm = (x * x).sum(1)
    nn = np.arange(n, dtype=np.int64)
    for base in range(0, n, block):
        e = min(n, base + block)
        if e - base < 2:
            continue
        for b0 in range(base, e, 4096):
            b1 = min(e, b0 + 4096)
            sc = 2 * x[b0:b1] @ x[base:e].T - nrm[None, base:e]
            r = torch.arange(b1 - b0)
            sc[r, r + b0 - base] = -float("inf")
            nn[b0:b1] = base + sc.argmax(1).numpy()    # the first of equal maxima
    p = nn.copy()
    reach = 1
    while reach < 2 * n:
        p = p[p]
        reach *= 2
    root = np.minimum(p, nn[p])
    return np.lexsort((np.arange(n), root, first[root] >> 4))


@pytest.mark.parametrize("case", ["select", "equal_latents", "one_query", "many"])
def test_grouped_attention_latent_order(tiny, case):
    """lsa_sparse_attn_grouped with the query latents: the order the prepare
    half leaves in the workspace equals the host statement of the latent
    nearest-neighbour order (index work, bit-exact), each group's union size
    equals the distinct long-range keys of its queries' rows, and the output
    matches the window kernel's (the two halves and the one call alike).
    Cases: the select's rows for 3000 queries; every query with the same
    latent (all nearest neighbours tie: the lowest index wins); one query;
    45000 queries on a 64k-key index (two blocks of the neighbour search:
    32768 queries, then 12232)."""
    wl, g, latk, ref, dev = tiny
    L = _L()
    Hq, Hkv, D = 8, 2, 64
    wl = dataclasses.replace(wl, Hq=Hq, Hkv=Hkv, D=D)
    if case == "many":
        wl = dataclasses.replace(wl, T=1 << 16)
    g = S.Synth(wl)
    if case == "many":
        latk = g.latk(0, wl.T)
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    nq = {"select": 3000, "equal_latents": 700, "one_query": 1, "many": 45000}[case]
    qpos0 = 12000 if case != "many" else 20000
    pos = torch.arange(qpos0, qpos0 + nq)
    lq = g.latq_rows(pos)
    if case == "equal_latents":
        lq = lq[:1].repeat(nq, 1).contiguous()
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    idx, cnt = ix.select(lq.to(dev), pos.to(torch.int32).to(dev), sp)
    q = g.q_rows(pos).to(dev)
    K = torch.empty((wl.T, Hkv, D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    K, V = K.to(dev), V.to(dev)
    ap32 = L.AttnParams(Hq, Hkv, D, 1, 0.0)
    lqd = lq.to(dev)
    ws = torch.zeros(L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap32, nq), dtype=torch.uint8,
                     device=dev)
    L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32, ws=ws, part="prepare", latq=lqd)
    torch.cuda.synchronize()
    qpw = 16 // (Hq // Hkv)
    perm, ucnt = _grouped_plan_from_ws(ws, nq, qpw, sp.budget)
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy().astype(np.int64)
    t = np.arange(qpos0, qpos0 + nq)
    wstart = np.maximum(0, t - wl.window + 1)
    lr = cnt_h - (np.maximum(0, np.minimum(wl.sinks, wstart)) + (t - wstart + 1))
    first = np.where(lr > 0, idx_h[:, 0].astype(np.int64), (1 << 28) - 1)
    order = _latent_order(lq.numpy(), first)
    assert np.array_equal(perm, order)
    sizes = [np.unique(np.concatenate([idx_h[j, :lr[j]] for j in order[g0:g0 + qpw]])).size
             for g0 in range(0, nq, qpw)]
    assert np.array_equal(ucnt, np.asarray(sizes, dtype=np.int32))
    halves = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32, ws=ws, part="walk")
    whole = L.sparse_attn_grouped(q, K, V, idx, cnt, qpos0, sp, ap32, latq=lqd)
    win = L.sparse_attn_window(q, K, V, idx, cnt, qpos0, sp, ap32)
    torch.cuda.synchronize()
    assert torch.equal(halves, whole)
    e = normwise(whole.cpu().numpy().astype(np.float64), win.cpu().numpy().astype(np.float64))
    print(f"{case}: latent-ordered grouped vs window kernel, {nq} queries: {e:.3e}; "
          f"unions {sum(sizes) / max(1, lr.sum()):.3f} of the long-range entries")
    assert e <= TOL


def test_grouped_attention_identical_rows():
    """Every query of a group holding the same long-range keys (each union
    row masked for all its queries), rows shorter than a tile, and queries
    with no long-range key at all (first positions)."""
    dev = _dev()
    L = _L()
    Hq, Hkv, D, budget, window, sinks = 8, 2, 64, 40, 16, 2
    wl = S.Workload("grp", 91, T=2048, ncomp=16, block=64, buckets=16, iters=2, chunk=0,
                    budget=budget, window=window, sinks=sinks, Hq=Hq, Hkv=Hkv, D=D)
    g = S.Synth(wl, data_cfg=91)
    qpos0, nq = 0, 300
    rng = np.random.default_rng(3)
    shared = [np.sort(rng.choice(800, size=int(rng.integers(1, budget + 1)), replace=False))
              for _ in range(8)]
    idx = torch.full((nq, wl.max_sel), -1, dtype=torch.int32)
    cnt = torch.zeros(nq, dtype=torch.int32)
    sels = []
    for i in range(nq):
        t = qpos0 + i
        ws = max(0, t - window + 1)
        ns = max(0, min(sinks, ws))
        fixed = list(range(ns)) + list(range(ws, t + 1))
        lr = [k for k in shared[(i // 37) % 8].tolist() if k < ws and k >= ns] if t >= 40 else []
        row = np.array(lr + fixed, dtype=np.int32)
        idx[i, :len(row)] = torch.from_numpy(row)
        cnt[i] = len(row)
        sels.append(np.sort(row.astype(np.int64)))
    pos = list(range(qpos0, qpos0 + nq))
    q = g.q_rows(torch.tensor(pos))
    K = torch.empty((wl.T, Hkv, D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    sp = L.SelectParams(budget, window, sinks, 0)
    o = L.sparse_attn_grouped(q.to(dev), K.to(dev), V.to(dev), idx.to(dev), cnt.to(dev), qpos0, sp,
                              L.AttnParams(Hq, Hkv, D, 1, 0.0))
    err = normwise(o.cpu().numpy().astype(np.float64), oracle_attention(g, wl, pos, sels))
    print(f"grouped attention, identical rows: {err:.3e}")
    assert err <= TOL


def test_grouped_attention_rejects():
    """Shapes the grouped kernel does not take are refused on the host."""
    _dev()
    L = _L()
    sp = L.SelectParams(4096, 512, 4, 0)
    for ap in (L.AttnParams(8, 8, 128, 0, 0.0), L.AttnParams(6, 2, 64, 0, 0.0),
               L.AttnParams(8, 1, 64, 0, 0.0)):
        n = 16
        q = torch.zeros((n, ap.Hq, ap.D), dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros((64, ap.Hkv, ap.D), dtype=torch.bfloat16, device="cuda")
        idx = torch.full((n, sp.max_sel), -1, dtype=torch.int32, device="cuda")
        cnt = torch.ones(n, dtype=torch.int32, device="cuda")
        if ap.Hq // ap.Hkv == 8:        # G = 8 with a 4096 budget: 2 x 4096 fits; G = 1, 3 do not
            L.sparse_attn_grouped(q, kv, kv, idx, cnt, 0, sp, ap)
            continue
        with pytest.raises(L.LsaError):
            L.sparse_attn_grouped(q, kv, kv, idx, cnt, 0, sp, ap)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_append_equals_build(seed):
    """Chunked and per-token appends (crossing tail re-clusters) equal a one-shot build."""
    dev = _dev()
    L = _L()
    wl = S.Workload("app", 90 + seed, T=4 * 256 * 5 + 37, ncomp=64, block=256, buckets=32,
                    iters=3, chunk=0, budget=200, window=64, sinks=4, Hq=4, Hkv=1, D=64)
    g = S.Synth(wl, data_cfg=90 + seed)
    latk = g.latk(0, wl.T)
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    ix = L.LsaIndex(_iparams(wl), dev)
    rng = np.random.default_rng(seed)
    cuts = sorted(set(rng.integers(1, wl.T, 12).tolist() + [1, 2, 3, 1024, 1025, 2048]))
    prev = 0
    for c in cuts + [wl.T]:
        ix.append(latk[prev:c].to(dev))
        prev = c
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    # one key at a time over a block boundary
    ix2 = L.LsaIndex(_iparams(wl), dev)
    ix2.build(latk[:1000].to(dev))
    for t in range(1000, 1100):
        ix2.append(latk[t:t + 1].to(dev))
    torch.cuda.synchronize()
    check_index(ix2.arrays(), O.build_index(latk.numpy(), 1100, _oparams(wl)))


def test_edge_cases_small_contexts_ties_budget0():
    dev = _dev()
    L = _L()
    wl = S.Workload("edge", 80, T=4 * 64 * 3 + 2, ncomp=8, block=64, buckets=16, iters=2,
                    chunk=0, budget=50, window=8, sinks=3, Hq=2, Hkv=2, D=64)
    g = S.Synth(wl, data_cfg=80)
    latk = g.latk(0, wl.T)
    latk[100:300] = 5                                   # exact duplicates -> distance ties
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    pos = [0, 1, 2, 7, 8, 10, 11, 12, 60, 200, wl.T - 1, wl.T - 2, 333]
    lq = g.latq_rows(torch.tensor(pos))
    lq[3] = 0                                          # every score ties
    for B in (0, 1, 7, 50, 400):
        sp = L.SelectParams(B, wl.window, wl.sinks, 0)
        osp = O.SelectParams(B, wl.window, wl.sinks)
        idx, cnt = ix.select(lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp)
        refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
        check_selection(idx, cnt, refs, sp.max_sel)
    # empty query batch
    idx, cnt = ix.select(lq[:0].to(dev), torch.zeros(0, dtype=torch.int32, device=dev),
                         L.SelectParams(10, 8, 3, 0))
    assert idx.shape == (0, 21)


def test_dense_select_matches_oracle():
    dev = _dev()
    L = _L()
    wl = S.WORKLOADS["tiny_flat"]
    g = S.Synth(wl)
    T = 6000
    latk = g.latk(0, T)
    pos = [5, 200, 1000, 2047, 4096, 5999, 3333, 4444, 5555, 130, 131]
    lq = g.latq_rows(torch.tensor(pos))
    sp = L.SelectParams(300, 128, 4, 0)
    osp = O.SelectParams(300, 128, 4)
    idx, cnt = L.dense_select(latk.to(dev), lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp)
    refs = [O.dense_select(latk.numpy(), lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, refs, sp.max_sel)


@pytest.mark.parametrize("early", [(0, 0), (150, 4000)])
def test_dense_select_scan_path(early):
    """The comparator's thresholded scan (batches of 64 or more queries with a
    workspace) against the oracle and against the exact kernel, with queries
    near the start of the context (lists that hold every eligible key) and
    the position-dependent budget switching inside the batch."""
    dev = _dev()
    L = _L()
    wl = S.WORKLOADS["tiny_flat"]
    g = S.Synth(wl)
    T = 12000
    latk = g.latk(0, T)
    rng = np.random.default_rng(81)
    pos = sorted(set([5, 130, 131, 600, 1100, 3999, 4000, 4001, T - 1] + rng.integers(0, T, 180).tolist()))
    lq = g.latq_rows(torch.tensor(pos))
    sp = L.SelectParams(300, 128, 4, 0, *early)
    osp = O.SelectParams(300, 128, 4, 0, *early)
    qp = torch.tensor(pos, dtype=torch.int32, device=dev)
    idx, cnt = L.dense_select(latk.to(dev), lq.to(dev), qp, sp)
    refs = [O.dense_select(latk.numpy(), lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, refs, sp.max_sel)
    idx2, cnt2 = L.dense_select(latk.to(dev), lq.to(dev), qp, sp, use_workspace=False)
    assert torch.equal(cnt, cnt2)
    for i in range(len(pos)):
        n = int(cnt[i])
        assert torch.equal(torch.sort(idx[i, :n]).values, torch.sort(idx2[i, :n]).values), pos[i]


def test_dense_select_scan_path_overflow():
    """Every latent key the same: all of a query's scores tie, every key
    passes its threshold and each of its key-range sub-lists overflows, so the
    exact kernel serves every query; ties go to the lowest positions."""
    dev = _dev()
    L = _L()
    T = 40000
    row = torch.arange(64, dtype=torch.int64).remainder(23).sub(11).to(torch.int8)
    latk = row.repeat(T, 1)
    wl = S.WORKLOADS["tiny_flat"]
    g = S.Synth(wl)
    rng = np.random.default_rng(7)
    pos = sorted(set(rng.integers(20000, T, 70).tolist()) | {T - 1})
    lq = g.latq_rows(torch.tensor(pos))
    sp = L.SelectParams(300, 128, 4, 0)
    osp = O.SelectParams(300, 128, 4)
    qp = torch.tensor(pos, dtype=torch.int32, device=dev)
    idx, cnt = L.dense_select(latk.to(dev), lq.to(dev), qp, sp)
    refs = [O.dense_select(latk.numpy(), lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
    check_selection(idx, cnt, refs, sp.max_sel)


@pytest.mark.parametrize("tree_iters", [3, 1])
def test_tree_index_and_selection(tree_iters):
    """Two-level Tree index and selections; the super level runs its own
    iteration count (equal to, then different from, the leaf level's)."""
    dev = _dev()
    L = _L()
    wl = S.Workload("tree_small", 70, T=4 * 256 * 12 + 300, ncomp=128, block=256, buckets=32,
                    iters=3, tree_group=4, tree_super=16, tree_iters=tree_iters, tree_top=5, chunk=0,
                    budget=500, window=64, sinks=4, Hq=4, Hkv=1, D=64)
    g = S.Synth(wl, data_cfg=70)
    latk = g.latk(0, wl.T)
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    assert ref.n_grp == 3
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    pos = [wl.T - 1 - 37 * i for i in range(40)] + [70, 500, 4000]
    lq = g.latq_rows(torch.tensor(pos))
    for R, eb, eu in ((1, 0, 0), (5, 0, 0), (48, 0, 0), (5, 120, 9000)):
        sp = L.SelectParams(wl.budget, wl.window, wl.sinks, R, eb, eu)
        osp = O.SelectParams(wl.budget, wl.window, wl.sinks, R, eb, eu)
        idx, cnt = ix.select(lq.to(dev), torch.tensor(pos, dtype=torch.int32, device=dev), sp)
        refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
        check_selection(idx, cnt, refs, sp.max_sel)


def test_tree_selection_at_extreme_scores():
    """Latent keys whose pooled vectors are all -128 or all 127, so leaf and
    super centroids sit at the int8 extremes, and queries of all -128 / all
    127 / mixed signs: scores reach 2^20 and -1040384, the ends of the range
    the Tree kernel packs into its 32-bit node keys, with many equal scores
    ordered by id."""
    dev = _dev()
    L = _L()
    wl = S.Workload("tree_extreme", 72, T=3 * 4 * 64 * 4 + 100, ncomp=64, block=64, buckets=16,
                    iters=3, tree_group=4, tree_super=16, tree_iters=3, tree_top=5, chunk=0,
                    budget=300, window=32, sinks=4, Hq=4, Hkv=1, D=64)
    rng = np.random.default_rng(72)
    sign = rng.integers(0, 2, size=(wl.T + wl.pool - 1) // wl.pool)     # per pooled group
    rows = np.where(np.repeat(sign, wl.pool)[:wl.T, None] == 1, 127, -128)
    latk = torch.from_numpy(np.broadcast_to(rows, (wl.T, 64)).astype(np.int8).copy())
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    assert ref.n_grp == 3
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    pos = [wl.T - 1, wl.T - 50, 2000, 900]
    qs = [np.full(64, -128), np.full(64, 127), np.where(np.arange(64) % 2 == 0, 127, -128),
          np.zeros(64)]
    lq = torch.from_numpy(np.stack([q for q in qs for _ in pos]).astype(np.int8))
    qpos = pos * len(qs)
    for R in (1, 5, 12):
        sp = L.SelectParams(wl.budget, wl.window, wl.sinks, R)
        osp = O.SelectParams(wl.budget, wl.window, wl.sinks, R)
        idx, cnt = ix.select(lq.to(dev), torch.tensor(qpos, dtype=torch.int32, device=dev), sp)
        refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(qpos)]
        check_selection(idx, cnt, refs, sp.max_sel)


TREE3 = S.Workload("tree3_small", 71, T=4 * 64 * 2 * 10 + 300, ncomp=96, block=64, buckets=32,
                   iters=3, tree_group=2, tree_super=16, tree_iters=3, tree_top=6, tree2_group=4,
                   tree2_super=16, tree2_iters=3, tree2_top=3, chunk=0, budget=300, window=64,
                   sinks=4, Hq=4, Hkv=1, D=64)
# the same shape with a different Lloyd iteration count on every level
TREE3_ITERS = dataclasses.replace(TREE3, name="tree3_iters", iters=3, tree_iters=1, tree2_iters=2)


@pytest.mark.parametrize("wl", [TREE3, TREE3_ITERS], ids=lambda w: w.name)
def test_tree3_index_and_selection(wl):
    """Three-level Tree: 10 groups of 2 blocks, top groups of 4 groups (2
    complete, 2 groups and a partial block outside them).  Index bit-exact,
    selections of the fast Tree kernel and of the exact kernel bit-exact."""
    dev = _dev()
    L = _L()
    g = S.Synth(wl, data_cfg=71)
    latk = g.latk(0, wl.T)
    ref = O.build_index(latk.numpy(), wl.T, _oparams(wl))
    assert ref.n_grp == 10 and ref.n_grp2 == 2 and ref.top_centroids.shape[0] == 32
    ix = L.LsaIndex(_iparams(wl), dev)
    ix.build(latk.to(dev))
    torch.cuda.synchronize()
    check_index(ix.arrays(), ref)
    pos = [wl.T - 1 - 41 * i for i in range(48)] + [70, 700, 3000, 6000]
    lq = g.latq_rows(torch.tensor(pos))
    qd = torch.tensor(pos, dtype=torch.int32, device=dev)
    for R, R2 in ((1, 1), (6, 3), (6, 8), (40, 2)):
        sp = L.SelectParams(wl.budget, wl.window, wl.sinks, R, 0, 0, R2)
        osp = O.SelectParams(wl.budget, wl.window, wl.sinks, R, tree2_top=R2)
        refs = [O.select(ref, lq[i].numpy(), t, osp) for i, t in enumerate(pos)]
        idx, cnt = ix.select(lq.to(dev), qd, sp)
        check_selection(idx, cnt, refs, sp.max_sel)
        idx2, cnt2 = ix.select(lq.to(dev), qd, sp, use_workspace=False)
        assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    with pytest.raises(L.LsaError, match="tree2_top"):
        ix.select(lq.to(dev), qd, L.SelectParams(wl.budget, wl.window, wl.sinks, 6))


@pytest.mark.parametrize("wl", [TREE3, TREE3_ITERS], ids=lambda w: w.name)
def test_tree3_append_equals_build_and_decode(wl):
    """Appending key by key across a top-group completion gives the built
    index; decode steps on two sequences select the oracle's keys."""
    dev = _dev()
    L = _L()
    kpt = wl.pool * wl.block * wl.tree_group * wl.tree2_group     # keys per top group
    Ts = [kpt - 2, 2 * kpt + 77]
    steps = 5
    cap = max(Ts) + steps
    gens = [S.Synth(wl, seq=i, data_cfg=72) for i in range(2)]
    ip = _iparams(wl, cap)
    op = _oparams(wl)
    K = torch.empty((2, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    ixs, lat = [], []
    for i, gg in enumerate(gens):
        lk = gg.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:Ts[i]].to(dev))
        ixs.append(ix)
        gg.fill_rows("k", K[i], 0)
        gg.fill_rows("v", V[i], 0)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, 0, 0, wl.tree2_top)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, tree2_top=wl.tree2_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, 2), dtype=torch.uint8,
                     device=dev)
    Kd, Vd = K.to(dev), V.to(dev)
    for step in range(steps):
        ts = [T + step for T in Ts]
        lk_new = torch.stack([lat[i][t] for i, t in enumerate(ts)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, 2, sp)
        torch.cuda.synchronize()
        for i, t in enumerate(ts):
            sel = O.select(O.build_index(lat[i].numpy(), t + 1, op), lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} step {step}"
    for i in range(2):
        full = O.build_index(lat[i].numpy(), Ts[i] + steps, op)
        check_index(ixs[i].arrays(), full)
    assert full.n_grp2 == 2


@pytest.mark.parametrize("early", [(0, 0), (100, 4 * 256 * 4 + 5 + 4)])
def test_decode_steps_match_oracle(early):
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_small", 60, T=4 * 256 * 4 + 5, ncomp=64, block=256, buckets=32, iters=3,
                    chunk=0, budget=300, window=64, sinks=4, Hq=8, Hkv=2, D=128, nseq=3, steps=9)
    gens = [S.Synth(wl, seq=i, data_cfg=60) for i in range(wl.nseq)]
    cap = wl.T + wl.steps
    ixs, lat = [], []
    K = torch.empty((wl.nseq, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(_iparams(wl, cap), dev)
        ix.build(lk[:wl.T].to(dev))
        ixs.append(ix)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0, *early)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, 0, *early)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    errs = []
    for step in range(wl.steps):
        t = wl.T + step
        lk_new = torch.stack([lat[i][t] for i in range(wl.nseq)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i in range(wl.nseq)])
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i in range(wl.nseq)])
        out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap)
        torch.cuda.synchronize()
        for i in range(wl.nseq):
            ref = O.build_index(lat[i].numpy(), t + 1, _oparams(wl))
            sel = O.select(ref, lq[i].numpy(), t, osp)
            ro = oracle_attention(gens[i], wl, [t], [sel])[0]
            errs.append(normwise(out[i].cpu().numpy().astype(np.float64), ro))
    check_index(ixs[0].arrays(), O.build_index(lat[0].numpy(), wl.T + wl.steps, _oparams(wl)))
    print("decode max normwise error", max(errs))
    assert max(errs) <= TOL


def test_decode_block_completes_mid_run():
    """Flat decode where one sequence's key completes a block (its append
    re-clusters the block) while the others in the batch take the one-key
    append inside the score kernel; index and selections match the oracle."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_blk", 65, T=0, ncomp=64, block=64, buckets=16, iters=3, chunk=0,
                    budget=150, window=24, sinks=2, Hq=4, Hkv=2, D=64)
    kpb = wl.pool * wl.block                          # keys per block
    Ts = [5 * kpb - 3, 3 * kpb + 37, 2 * kpb]         # seq 0 completes block 5 at its third key
    steps = 7
    cap = max(Ts) + steps
    gens = [S.Synth(wl, seq=i, data_cfg=65) for i in range(len(Ts))]
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap)
    op = _oparams(wl)
    K = torch.empty((len(Ts), cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    ixs, lat = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:Ts[i]].to(dev))
        ixs.append(ix)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, len(Ts)), dtype=torch.uint8,
                     device=dev)
    for step in range(steps):
        ts = [T + step for T in Ts]
        lk_new = torch.stack([lat[i][t] for i, t in enumerate(ts)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, len(Ts), sp)
        torch.cuda.synchronize()
        for i, t in enumerate(ts):
            sel = O.select(O.build_index(lat[i].numpy(), t + 1, op), lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} step {step}"
            err = normwise(out[i].cpu().numpy().astype(np.float64),
                           oracle_attention(gens[i], wl, [t], [sel])[0])
            assert err <= TOL, (i, step, err)
    assert ixs[0].info().n_full == 5
    for i in range(len(Ts)):
        check_index(ixs[i].arrays(), O.build_index(lat[i].numpy(), Ts[i] + steps, op))


def test_decode_sixteen_sequences():
    """The largest decode batch: 16 sequences of different lengths."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec16", 62, T=0, ncomp=32, block=64, buckets=16, iters=2, chunk=0,
                    budget=120, window=32, sinks=2, Hq=4, Hkv=2, D=64)
    Ts = [300 + 157 * i for i in range(16)]
    steps = 3
    cap = max(Ts) + steps
    gens = [S.Synth(wl, seq=i, data_cfg=62) for i in range(16)]
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap)
    op = _oparams(wl)
    K = torch.empty((16, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    ixs, lat = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:Ts[i]].to(dev))
        ixs.append(ix)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, 16), dtype=torch.uint8,
                     device=dev)
    errs = []
    for step in range(steps):
        ts = [T + step for T in Ts]
        lk_new = torch.stack([lat[i][t] for i, t in enumerate(ts)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, 16, sp)
        torch.cuda.synchronize()
        for i, t in enumerate(ts):
            sel = O.select(O.build_index(lat[i].numpy(), t + 1, op), lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} step {step}"
            errs.append(normwise(out[i].cpu().numpy().astype(np.float64),
                                 oracle_attention(gens[i], wl, [t], [sel])[0]))
    assert max(errs) <= TOL
    with pytest.raises(L.LsaError, match="nseq"):
        L.decode_step(ixs + ixs[:1], torch.zeros((17, 64), dtype=torch.int8, device=dev),
                      torch.zeros((17, 64), dtype=torch.int8, device=dev),
                      torch.zeros((17, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev), Kd, Vd, cap,
                      sp, ap, ws=ws)


def test_decode_tied_scores_and_small_budgets():
    """Decode with every score tied (a zero latent query: one score bin holds
    all 322 buckets, more than the cutoff bin a direct ranking takes), budgets
    of 0, 7, 150 and one above every eligible key, next to an ordinary query."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_ties", 63, T=4 * 64 * 20 + 11, ncomp=16, block=64, buckets=16, iters=2,
                    chunk=0, budget=150, window=16, sinks=2, Hq=4, Hkv=2, D=64)
    gens = [S.Synth(wl, seq=i, data_cfg=63) for i in range(2)]
    cap = wl.T + 1
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap)
    op = _oparams(wl)
    K = torch.empty((2, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    lat = [g.latk(0, cap) for g in gens]
    for i, g in enumerate(gens):
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    t = wl.T
    lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i in range(2)])
    lq[0] = 0
    q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i in range(2)])
    lk_new = torch.stack([lat[i][t] for i in range(2)])
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    for budget in (0, 7, 150, 4096):
        ixs = []
        for i in range(2):
            ix = L.LsaIndex(ip, dev)
            ix.build(lat[i][:t].to(dev))
            ixs.append(ix)
        sp = L.SelectParams(budget, wl.window, wl.sinks, 0)
        osp = O.SelectParams(budget, wl.window, wl.sinks)
        ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, 2), dtype=torch.uint8,
                         device=dev)
        L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, 2, sp)
        torch.cuda.synchronize()
        for i in range(2):
            sel = O.select(O.build_index(lat[i].numpy(), t + 1, op), lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} budget {budget}"


def test_decode_large_indexes():
    """Decode over indexes of about 19k, 22k and 25.6k buckets: 24 buckets per
    select thread, 19 and 22 partial score histograms (not multiples of four),
    past 24576 buckets the streaming kernel (alone, and in a batch beside a
    register-resident sequence), and a zero latent query on the large index
    (every score tied: the exact kernel, one sequence at its own position)."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_large", 64, T=0, ncomp=128, block=64, buckets=32, iters=2, chunk=0,
                    budget=512, window=64, sinks=4, Hq=4, Hkv=2, D=64)
    steps = 2
    # full blocks of 64 pooled vectors give 32 buckets each; tails are singletons
    # the last: 32776 buckets, not a multiple of the streaming kernel's 8192-bucket
    # batch, so its final batch is partial for every lane but the first few
    Ts = [4 * 64 * 594 + 4 * 17 + 1, 4 * 64 * 687 + 4 * 40 + 3, 4 * 64 * 800 + 11, 4 * 64 * 1024 + 4 * 8 + 1]
    nbk = [594 * 32 + 17, 687 * 32 + 40, 800 * 32 + 2, 1024 * 32 + 8]
    assert nbk[0] <= 20480 < nbk[1] <= 24576 < nbk[2] < nbk[3]
    cap = max(Ts) + steps
    op = _oparams(wl)
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap)
    gens = [S.Synth(wl, seq=i, data_cfg=64) for i in range(4)]
    lat = [g.latk(0, cap) for g in gens]
    K = torch.empty((4, cap, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for i, g in enumerate(gens):
        g.fill_rows("k", K[i], 0, chunk=1 << 16)
        g.fill_rows("v", V[i], 0, chunk=1 << 16)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    caches = [dict() for _ in range(4)]
    for batch in ([0, 1], [2], [1, 2], [3]):
        ixs = []
        for i in batch:
            ix = L.LsaIndex(ip, dev)
            ix.build(lat[i][:Ts[i]].to(dev))
            assert ix.info().n_bkt == nbk[i]
            ixs.append(ix)
        # one K/V cache per batch: the sequences of a decode step are rows of one tensor
        Kb, Vb = K[batch].contiguous(), V[batch].contiguous()
        ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, len(batch)),
                         dtype=torch.uint8, device=dev)
        for step in range(steps):
            ts = [Ts[i] + step for i in batch]
            lk_new = torch.stack([lat[i][t] for i, t in zip(batch, ts)])
            lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in zip(batch, ts)])
            if batch == [2] and step == 1:
                lq.zero_()
            q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in zip(batch, ts)])
            print(f"decode batch {batch} step {step}", flush=True)
            out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kb, Vb, cap, sp, ap, ws=ws)
            idx, cnt = L.decode_selection(ws, len(batch), sp)
            torch.cuda.synchronize()
            for b, (i, t) in enumerate(zip(batch, ts)):
                ref = O.build_index(lat[i].numpy(), t + 1, op, cache=caches[i])
                sel = O.select(ref, lq[b].numpy(), t, osp)
                n = int(cnt[b])
                assert np.array_equal(np.sort(idx[b, :n].cpu().numpy()), sel), f"seq {i} step {step}"
                err = normwise(out[b].cpu().numpy().astype(np.float64),
                               oracle_attention(gens[i], wl, [t], [sel])[0])
                assert err <= TOL, (i, step, err)


def test_tree_decode_steps_match_oracle():
    """Decode on Tree indexes: sequences of different lengths, one without a
    complete group until its third step (its super level is built during
    decode), one whose block completes mid-run."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_tree", 61, T=0, ncomp=64, block=64, buckets=16, iters=3, tree_group=4,
                    tree_super=16, tree_iters=2, tree_top=5, chunk=0, budget=200, window=32,
                    sinks=4, Hq=8, Hkv=2, D=64)
    kpg = wl.pool * wl.block * wl.tree_group           # keys per group
    Ts = [kpg - 3, 2 * kpg + 500, 3 * kpg - 130]
    steps = 9
    cap = max(Ts) + steps
    gens = [S.Synth(wl, seq=i, data_cfg=61) for i in range(len(Ts))]
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group, wl.tree_super,
                       wl.tree_iters, cap)
    op = _oparams(wl)
    K = torch.empty((len(Ts), cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    ixs, lat = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:Ts[i]].to(dev))
        ixs.append(ix)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, len(Ts)), dtype=torch.uint8,
                     device=dev)
    errs = []
    for step in range(steps):
        ts = [T + step for T in Ts]
        lk_new = torch.stack([lat[i][t] for i, t in enumerate(ts)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, len(Ts), sp)
        torch.cuda.synchronize()
        for i, t in enumerate(ts):
            ref = O.build_index(lat[i].numpy(), t + 1, op)
            sel = O.select(ref, lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} step {step}"
            ro = oracle_attention(gens[i], wl, [t], [sel])[0]
            errs.append(normwise(out[i].cpu().numpy().astype(np.float64), ro))
    for i in range(len(Ts)):
        check_index(ixs[i].arrays(), O.build_index(lat[i].numpy(), Ts[i] + steps, op))
    assert max(errs) <= TOL


def test_single_sequence_tree_decode_with_tied_scores():
    """One sequence on a Tree index, first with a zero latent query (every
    score tied), then an ordinary one: ties send the sequence to the exact
    refinement, which must serve a batch of one at its own position."""
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_tree1", 61, T=0, ncomp=64, block=64, buckets=16, iters=3, tree_group=4,
                    tree_super=16, tree_iters=3, tree_top=5, chunk=0, budget=200, window=32,
                    sinks=4, Hq=8, Hkv=2, D=64)
    T0 = 2 * wl.pool * wl.block * wl.tree_group + 500
    cap = T0 + 2
    g = S.Synth(wl, seq=0, data_cfg=61)
    ip = L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, wl.tree_group, wl.tree_super,
                       wl.tree_iters, cap)
    lat = g.latk(0, cap)
    ix = L.LsaIndex(ip, dev)
    ix.build(lat[:T0].to(dev))
    K = torch.empty((1, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K[0], 0)
    g.fill_rows("v", V[0], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, 1), dtype=torch.uint8,
                     device=dev)
    for step in range(2):
        t = T0 + step
        lq = g.latq_rows(torch.tensor([t]))
        if step == 0:
            lq.zero_()
        q = g.q_rows(torch.tensor([t]))
        out = L.decode_step([ix], lat[t:t + 1].to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap,
                            ws=ws)
        idx, cnt = L.decode_selection(ws, 1, sp)
        torch.cuda.synchronize()
        sel = O.select(O.build_index(lat.numpy(), t + 1, _oparams(wl)), lq[0].numpy(), t, osp)
        n = int(cnt[0])
        assert np.array_equal(np.sort(idx[0, :n].cpu().numpy()), sel), f"step {step}"
        err = normwise(out[0].cpu().numpy().astype(np.float64),
                       oracle_attention(g, wl, [t], [sel])[0])
        assert err <= TOL, (step, err)


@pytest.mark.parametrize("levels", [2, 3])
def test_tree_decode_candidate_overflow(levels):
    """Tree decode where the chosen supers hold many leaves (two levels: 72
    of 96 supers, about 5000 leaves, beyond the Tree kernel's candidate list;
    three levels: the best 40 of the 12 supers under the 4 best of 16 top nodes
    and the 32 supers under no top node, about 2400 leaves): that sequence
    goes through the streaming pair restricted to its candidates, batched with
    a sequence the Tree kernel serves; a zero query (every score tied) then
    falls through to the exact kernel."""
    dev = _dev()
    L = _L()
    t2 = dict(tree2_group=4, tree2_super=16, tree2_iters=1, tree2_top=4) if levels == 3 else {}
    wl = S.Workload("dec_tree_ovf", 71, T=0, ncomp=64, block=64, buckets=16, iters=3, tree_group=64,
                    tree_super=16, tree_iters=2, tree_top=72 if levels == 2 else 40, chunk=0,
                    budget=1500, window=32, sinks=4, Hq=8, Hkv=2, D=64, **t2)
    kpg = wl.pool * wl.block * wl.tree_group           # keys per group
    Ts = [6 * kpg + 300, kpg + 500]
    steps = 3
    cap = max(Ts) + steps
    gens = [S.Synth(wl, seq=i, data_cfg=71) for i in range(len(Ts))]
    ip = _iparams(wl, cap)
    op = _oparams(wl)
    K = torch.empty((len(Ts), cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    ixs, lat = [], []
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        ix = L.LsaIndex(ip, dev)
        ix.build(lk[:Ts[i]].to(dev))
        ixs.append(ix)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, 0, 0, wl.tree2_top)
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, wl.tree_top, tree2_top=wl.tree2_top)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    ws = torch.empty(L.workspace_bytes(L.binding.OP_DECODE, ip, sp, ap, len(Ts)), dtype=torch.uint8,
                     device=dev)
    errs = []
    for step in range(steps):
        ts = [T + step for T in Ts]
        lk_new = torch.stack([lat[i][t] for i, t in enumerate(ts)])
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        if step == 0:
            lq[0].zero_()
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i, t in enumerate(ts)])
        print(f"tree overflow decode step {step}", flush=True)
        out = L.decode_step(ixs, lk_new.to(dev), lq.to(dev), q.to(dev), Kd, Vd, cap, sp, ap, ws=ws)
        idx, cnt = L.decode_selection(ws, len(Ts), sp)
        torch.cuda.synchronize()
        for i, t in enumerate(ts):
            ref = O.build_index(lat[i].numpy(), t + 1, op)
            sel = O.select(ref, lq[i].numpy(), t, osp)
            n = int(cnt[i])
            assert np.array_equal(np.sort(idx[i, :n].cpu().numpy()), sel), f"seq {i} step {step}"
            ro = oracle_attention(gens[i], wl, [t], [sel])[0]
            errs.append(normwise(out[i].cpu().numpy().astype(np.float64), ro))
    assert max(errs) <= TOL


def test_api_errors_leave_index_unchanged(tiny):
    wl, g, latk, ref, dev = tiny
    L = _L()
    ix = L.LsaIndex(_iparams(wl, 4096), dev)
    ix.build(latk[:4000].to(dev))
    before = ix.snapshot()
    with pytest.raises(L.LsaError, match="capacity"):
        ix.append(latk[4000:4200].to(dev))
    assert ix.snapshot() == before
    with pytest.raises(L.LsaError):
        ix.select(latk[:2].to(dev), torch.zeros(2, dtype=torch.int32, device=dev),
                  L.SelectParams(5000, 8, 0, 0))
    assert ix.info().T == 4000
