"""The seeded input generators: determinism, row addressability, recipe stats."""
import numpy as np
import torch

import lsa_synth as S


def test_rows_regenerate_bit_identically():
    g = S.Synth(S.WORKLOADS["flat_1m"])
    a = g.latk(5000, 5100)
    b = g.latk_rows(torch.tensor([5000 + i for i in range(100)]))
    assert torch.equal(a, b)
    v = torch.empty((64, 8, 128), dtype=torch.bfloat16)
    g.fill_rows("v", v, 777)
    w = g.v_rows(torch.arange(777, 777 + 64))
    assert torch.equal(v.view(torch.int16), w.view(torch.int16))
    assert torch.equal(g.latq(10, 20), S.Synth(S.WORKLOADS["flat_1m"]).latq(10, 20))


def test_streams_and_sequences_differ():
    wl = S.WORKLOADS["decode_1m"]
    a, b = S.Synth(wl, seq=0), S.Synth(wl, seq=1)
    assert not torch.equal(a.latk(0, 64), b.latk(0, 64))
    assert not torch.equal(a.k_rows(torch.arange(4)).view(torch.int16),
                           a.v_rows(torch.arange(4)).view(torch.int16))


def test_tree_workload_shares_flat_10m_data():
    a = S.Synth(S.WORKLOADS["flat_10m"]).latk(123, 200)
    b = S.Synth(S.WORKLOADS["tree_10m"]).latk(123, 200)
    assert torch.equal(a, b)


def test_recipe_statistics():
    wl = S.WORKLOADS["tiny_flat"]
    g = S.Synth(wl)
    m = g.means64()
    assert m.shape == (256, 64) and m.min() >= -40 * 64 and m.max() <= 40 * 64
    lk = g.latk(0, 8192).float()
    assert lk.abs().max() <= 127
    q = g.k_rows(torch.arange(0, 4096)).float()
    assert abs(q.mean()) < 0.02 and abs(q.std() - 1.0) < 0.02
    t = S.normal_bf16_table().view(torch.bfloat16).float().numpy()
    assert np.all(np.diff(t) >= 0) and t[0] < -4.3 and t[-1] > 4.3
