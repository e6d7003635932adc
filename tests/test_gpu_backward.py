"""GPU parity of the training path: forward with log-sum-exp, and the sparse
attention backward (dQ, dK, dV) over the rows the select wrote, against the
float64 oracle over the oracle's own selections.

Every position of a short sequence is a query (a training step of one
layer), so the long-range, window and sink parts of dK / dV all occur, over
several key tiles and a ragged tail.  Gradients are float32; the bar is the
attention bar: 2e-3 normwise (max |gpu - ref| / max |ref| per tensor).
"""
import numpy as np
import pytest
import torch

import lsa_synth as S
import oracle as O
from test_gpu_parity import TOL, check_selection, normwise

pytestmark = pytest.mark.gpu


def _L():
    import hierarchical_sparse_attention_lsa_amd as L
    return L


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _f64(t):
    return O.bf16_to_f64(t.cpu().view(torch.int16).numpy())


def _setup(wl, dev, early=(0, 0), qpos0=0):
    """Index over all T keys, selection for queries qpos0..T-1, Q/K/V/dO."""
    L = _L()
    g = S.Synth(wl)
    T = wl.T
    latk = g.latk(0, T)
    ix = L.LsaIndex(L.IndexParams(64, wl.pool, wl.block, wl.buckets, wl.iters, 0, 0, 0, T), dev)
    ix.build(latk.to(dev))
    sp = L.SelectParams(wl.budget, wl.window, wl.sinks, 0, *early)
    pos = torch.arange(qpos0, T)
    lq = g.latq_rows(pos)
    idx, cnt = ix.select(lq.to(dev), pos.to(torch.int32).to(dev), sp)
    K = torch.empty((T, wl.Hkv, wl.D), dtype=torch.bfloat16)
    V = torch.empty_like(K)
    g.fill_rows("k", K, 0)
    g.fill_rows("v", V, 0)
    q = g.q_rows(pos)
    do = g.do_rows(pos)
    return dict(g=g, latk=latk, ix=ix, sp=sp, pos=pos.tolist(), lq=lq, idx=idx, cnt=cnt, K=K, V=V,
                q=q, do=do)


def _oracle(wl, r, early=(0, 0)):
    ref = O.build_index(r["latk"].numpy(), wl.T, O.IndexParams(wl.pool, wl.block, wl.buckets,
                                                                wl.iters))
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks, 0, *early)
    sels = [O.select(ref, r["lq"][i].numpy(), t, osp) for i, t in enumerate(r["pos"])]
    Kc, Vc = _f64(r["K"]), _f64(r["V"])
    Q, dO = _f64(r["q"]), _f64(r["do"])
    fw = [O.attend_lse(Q[i], Kc[s], Vc[s], wl.Hkv) for i, s in enumerate(sels)]
    lse = np.stack([f[1] for f in fw])
    # float32 stored output: the exact gradients; bf16 stored output: the
    # row sums dO . O come from the output rounded to bf16
    grads = {1: O.sparse_attention_backward(Q, Kc, Vc, dO, sels, wl.Hkv),
             0: O.sparse_attention_backward(Q, Kc, Vc, dO, sels, wl.Hkv,
                                            O=O.round_bf16(np.stack([f[0] for f in fw])))}
    return sels, lse, grads


CASES = [
    # name, workload, early budget
    ("d64_g2", S.Workload("bwd_a", 90, T=4 * 64 * 5 + 37, ncomp=12, block=64, buckets=16, iters=2,
                          chunk=0, budget=100, window=32, sinks=4, Hq=4, Hkv=2, D=64), (0, 0)),
    ("d128_g4_nosinks", S.Workload("bwd_b", 91, T=4 * 128 * 4 + 301, ncomp=20, block=128,
                                   buckets=32, iters=3, chunk=0, budget=250, window=64, sinks=0,
                                   Hq=8, Hkv=2, D=128), (0, 0)),
    ("d64_g3_early", S.Workload("bwd_c", 92, T=2 * 64 * 6 + 5, ncomp=8, block=64, buckets=16,
                                iters=2, chunk=0, budget=80, window=16, sinks=2, Hq=3, Hkv=1, D=64),
     (20, 400)),
    # G = 1 (16 queries per column group) and G = 16 (one), window = pool
    ("d128_g1", S.Workload("bwd_d", 93, T=4 * 64 * 3 + 70, ncomp=10, block=64, buckets=16,
                           iters=2, chunk=0, budget=64, window=4, sinks=1, Hq=4, Hkv=4, D=128),
     (0, 0)),
    ("d64_g16", S.Workload("bwd_e", 94, T=4 * 64 * 3 + 9, ncomp=10, block=64, buckets=16,
                           iters=2, chunk=0, budget=90, window=24, sinks=3, Hq=16, Hkv=1, D=64),
     (0, 0)),
]


@pytest.mark.parametrize("name,wl,early", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, wl, early):
    dev = _dev()
    L = _L()
    r = _setup(wl, dev, early)
    sels, lse_ref, grads = _oracle(wl, r, early)
    check_selection(r["idx"], r["cnt"], sels, r["sp"].max_sel)
    args = [t.to(dev) for t in (r["q"], r["K"], r["V"])]
    do = r["do"].to(dev)
    for out_f32 in (1, 0):
        ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, out_f32, 0.0)
        out, lse = L.sparse_attn_fwd(*args, r["idx"], r["cnt"], 0, r["sp"], ap)
        assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-4
        dq, dk, dv = L.sparse_attn_bwd(r["ix"], *args, r["idx"], r["cnt"], 0, r["sp"], ap, out, lse,
                                       do)
        torch.cuda.synchronize()
        dQ, dK, dV = grads[out_f32]
        errs = [normwise(x.cpu().numpy().astype(np.float64), y)
                for x, y in ((dq, dQ), (dk, dK), (dv, dV))]
        print(f"{name} out_f32={out_f32}: dQ/dK/dV normwise errors "
              + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) <= TOL
        # keys nobody selected (none here: every key is in some window) and
        # determinism: a second run is bitwise identical
        dq2, dk2, dv2 = L.sparse_attn_bwd(r["ix"], *args, r["idx"], r["cnt"], 0, r["sp"], ap, out,
                                          lse, do)
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


GROUPED_CASES = [c for c in CASES if (c[1].Hq // c[1].Hkv) in (4, 8, 16)]


@pytest.mark.parametrize("name,wl,early", GROUPED_CASES, ids=[c[0] for c in GROUPED_CASES])
def test_grouped_forward_for_training(name, wl, early):
    """The grouped attention as the training forward: its log-sum-exp and
    output against the oracle's, and the backward taken from them.  The bf16
    pass orders the groups (forward and dQ) by the query latents."""
    dev = _dev()
    L = _L()
    r = _setup(wl, dev, early)
    sels, lse_ref, grads = _oracle(wl, r, early)
    args = [t.to(dev) for t in (r["q"], r["K"], r["V"])]
    do = r["do"].to(dev)
    for out_f32 in (1, 0):
        ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, out_f32, 0.0)
        lse = torch.empty((len(r["pos"]), wl.Hq), dtype=torch.float32, device=dev)
        lat = r["lq"].to(dev) if not out_f32 else None
        out = L.sparse_attn_grouped(*args, r["idx"], r["cnt"], 0, r["sp"], ap, lse=lse, latq=lat)
        out_w, lse_w = L.sparse_attn_fwd(*args, r["idx"], r["cnt"], 0, r["sp"], ap)
        torch.cuda.synchronize()
        assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-4
        if out_f32:
            assert normwise(out.cpu().numpy().astype(np.float64),
                            out_w.cpu().numpy().astype(np.float64)) <= TOL
        dq, dk, dv = L.sparse_attn_bwd(r["ix"], *args, r["idx"], r["cnt"], 0, r["sp"], ap, out, lse,
                                       do, latq=lat)
        torch.cuda.synchronize()
        dQ, dK, dV = grads[out_f32]
        errs = [normwise(x.cpu().numpy().astype(np.float64), y)
                for x, y in ((dq, dQ), (dk, dK), (dv, dV))]
        print(f"{name} grouped forward, out_f32={out_f32}: dQ/dK/dV normwise errors "
              + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) <= TOL


def test_backward_of_a_suffix_and_unselected_keys():
    """Queries at positions qpos0.. only (a chunk), so keys after the last
    query get zero gradient and early keys get only the long-range and sink
    terms of the chunk's queries."""
    dev = _dev()
    L = _L()
    wl = CASES[0][1]
    qpos0 = 700
    r = _setup(wl, dev, qpos0=qpos0)
    ref = O.build_index(r["latk"].numpy(), wl.T, O.IndexParams(wl.pool, wl.block, wl.buckets,
                                                                wl.iters))
    osp = O.SelectParams(wl.budget, wl.window, wl.sinks)
    sels = [O.select(ref, r["lq"][i].numpy(), t, osp) for i, t in enumerate(r["pos"])]
    Kc, Vc = _f64(r["K"]), _f64(r["V"])
    dQ, dK, dV = O.sparse_attention_backward(_f64(r["q"]), Kc, Vc, _f64(r["do"]), sels, wl.Hkv)
    # the K/V cache holds 40 more rows than the index; they get zero
    K2 = torch.cat([r["K"], r["K"][:40]]).to(dev)
    V2 = torch.cat([r["V"], r["V"][:40]]).to(dev)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    q, do = r["q"].to(dev), r["do"].to(dev)
    out, lse = L.sparse_attn_fwd(q, K2, V2, r["idx"], r["cnt"], qpos0, r["sp"], ap)
    dq, dk, dv = L.sparse_attn_bwd(r["ix"], q, K2, V2, r["idx"], r["cnt"], qpos0, r["sp"], ap, out,
                                   lse, do)
    torch.cuda.synchronize()
    dk, dv = dk.cpu().numpy(), dv.cpu().numpy()
    assert (dk[wl.T:] == 0).all() and (dv[wl.T:] == 0).all()
    for x, y in ((dq.cpu().numpy(), dQ), (dk[:wl.T], dK), (dv[:wl.T], dV)):
        assert normwise(x.astype(np.float64), y) <= TOL
    never = np.setdiff1d(np.arange(wl.T), np.concatenate(sels))
    assert len(never) > 0
    assert (dk[never] == 0).all() and (dv[never] == 0).all()


def test_empty_batches():
    dev = _dev()
    L = _L()
    wl = CASES[0][1]
    r = _setup(wl, dev)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 1, 0.0)
    K, V = r["K"].to(dev), r["V"].to(dev)
    z = lambda *sh, dt=torch.bfloat16: torch.zeros(sh, dtype=dt, device=dev)
    idx0 = z(0, r["sp"].max_sel, dt=torch.int32)
    cnt0 = z(0, dt=torch.int32)
    out, lse = L.sparse_attn_fwd(z(0, wl.Hq, wl.D), K, V, idx0, cnt0, 5, r["sp"], ap)
    assert out.shape == (0, wl.Hq, wl.D) and lse.shape == (0, wl.Hq)
    dq, dk, dv = L.sparse_attn_bwd(r["ix"], z(0, wl.Hq, wl.D), K, V, idx0, cnt0, 5, r["sp"], ap,
                                   out, lse, z(0, wl.Hq, wl.D))
    assert dq.shape == (0, wl.Hq, wl.D)


def test_backward_rejects_bad_arguments():
    dev = _dev()
    L = _L()
    wl = CASES[0][1]
    r = _setup(wl, dev)
    ap = L.AttnParams(wl.Hq, wl.Hkv, wl.D, 0, 0.0)
    args = [t.to(dev) for t in (r["q"], r["K"], r["V"])]
    out, lse = L.sparse_attn_fwd(*args, r["idx"], r["cnt"], 0, r["sp"], ap)
    do = r["do"].to(dev)
    with pytest.raises(L.LsaError, match="workspace"):
        L.sparse_attn_bwd(r["ix"], *args, r["idx"], r["cnt"], 0, r["sp"], ap, out, lse, do,
                          ws=torch.empty(1024, dtype=torch.uint8, device=dev))
    sp_many = L.SelectParams(wl.budget, wl.window, 65, 0)
    with pytest.raises(L.LsaError, match="sinks"):
        L.sparse_attn_bwd(r["ix"], *args, torch.zeros((wl.T, sp_many.max_sel), dtype=torch.int32,
                                                      device=dev),
                          r["cnt"], 0, sp_many, ap, out, lse, do)
    with pytest.raises(L.LsaError, match="beyond"):
        L.sparse_attn_bwd(r["ix"], args[0][1:], args[1], args[2], r["idx"][1:], r["cnt"][1:], 2,
                          r["sp"], ap, out[1:], lse[1:], do[1:])
