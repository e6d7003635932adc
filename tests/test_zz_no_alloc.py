"""The no-allocation decode entry point against lsa_decode_step.

lsa_decode_step_noalloc runs the decode step in the library's own device
array instead of a caller workspace.  Through the C ABI, two sets of
identical indexes take the same keys and queries, one set through each entry
point, on two calls in a row (the second with fewer sequences): the outputs
must be bit-identical and the indexes must end up identical.  A step that
needs more workspace than the array holds is refused before anything is
enqueued.
"""

import pytest
import torch

import lsa_synth as S

pytestmark = pytest.mark.gpu


def _L():
    import hierarchical_sparse_attention_lsa_amd as L
    return L


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _params(L, wl, cap):
    return L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, cap)


def test_noalloc_decode_matches_decode_step():
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_noalloc", 62, T=4 * 256 * 4 + 3, ncomp=64, block=256, buckets=32, iters=3,
                    chunk=0, budget=300, window=64, sinks=4, Hq=8, Hkv=2, D=128, nseq=3, steps=2)
    cap = wl.T + wl.steps
    gens = [S.Synth(wl, seq=i, data_cfg=62) for i in range(wl.nseq)]
    K = torch.empty((wl.nseq, cap, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    lat = []
    sets = ([], [])
    for i, g in enumerate(gens):
        lk = g.latk(0, cap)
        lat.append(lk)
        g.fill_rows("k", K[i], 0)
        g.fill_rows("v", V[i], 0)
        for ixs in sets:
            ix = L.LsaIndex(_params(L, wl, cap), dev)
            ix.build(lk[:wl.T].to(dev))
            ixs.append(ix)
    Kd, Vd = K.to(dev), V.to(dev)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    assert L.lib().lsa_decode_step_noalloc_max_bytes() == 128 << 20
    # the stated coverage: 16 sequences of 10 * 2^20 keys at 4096 + 512 + 4, GQA 32/8, D = 128
    big = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 10 * 2 ** 20 + 256)
    need = L.workspace_bytes(L.binding.OP_DECODE, big, L.SelectParams(4096, 512, 4, 0),
                             L.AttnParams(32, 8, 128, 0, 0.0), 16)
    assert need <= L.lib().lsa_decode_step_noalloc_max_bytes()
    # call 1: all three sequences; call 2: a smaller batch (sequences 0 and 2)
    for step, members in ((0, [0, 1, 2]), (1, [0, 2])):
        t = wl.T + step
        n = len(members)
        lk_new = torch.stack([lat[i][t] for i in members]).to(dev)
        lq = torch.stack([gens[i].latq_rows(torch.tensor([t]))[0] for i in members]).to(dev)
        q = torch.stack([gens[i].q_rows(torch.tensor([t]))[0] for i in members]).to(dev)
        kk, vv = Kd[members].contiguous(), Vd[members].contiguous()
        print(f"no-alloc decode: call {step + 1}, {n} sequences at position {t}", flush=True)
        ref = L.decode_step([sets[0][i] for i in members], lk_new, lq, q, kk, vv, cap, sp, ap)
        out = torch.full((n, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        got = L.decode_step_noalloc([sets[1][i] for i in members], lk_new, lq, q, kk, vv, cap, sp, ap,
                                    out)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"call {step + 1}"
    for a, b in zip(*sets):
        assert a.info().T == b.info().T
        ga, gb = a.arrays(), b.arrays()
        for k in ga:
            assert torch.equal(ga[k], gb[k]), k


def test_noalloc_decode_refuses_an_oversized_step():
    dev = _dev()
    L = _L()
    wl = S.Workload("dec_noalloc_big", 63, T=600, ncomp=16, block=64, buckets=16, iters=2, chunk=0,
                    budget=64, window=1 << 20, sinks=4, Hq=16, Hkv=16, D=128, nseq=16, steps=1)
    g = S.Synth(wl, seq=0, data_cfg=63)
    lk = g.latk(0, wl.T + 1)
    ixs = []
    for _ in range(wl.nseq):
        ix = L.LsaIndex(_params(L, wl, wl.T + 1), dev)
        ix.build(lk[:wl.T].to(dev))
        ixs.append(ix)
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    need = L.workspace_bytes(L.binding.OP_DECODE, ixs[0].params, sp, ap, wl.nseq)
    assert need > L.lib().lsa_decode_step_noalloc_max_bytes()
    K = torch.zeros((wl.nseq, wl.T + 1, wl.Hkv, wl.D), dtype=torch.bfloat16, device=dev)
    rows = torch.stack([lk[wl.T]] * wl.nseq).to(dev)
    q = torch.zeros((wl.nseq, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((wl.nseq, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    with pytest.raises(L.LsaError, match="no-allocation"):
        L.decode_step_noalloc(ixs, rows, rows, q, K, K, wl.T + 1, sp, ap, out)
    torch.cuda.synchronize()
    assert all(ix.info().T == wl.T for ix in ixs)
    assert b"holds" in L.lib().lsa_last_error()
