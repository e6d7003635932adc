"""Pins of the oracle's sparse-attention backward, independent of its formulas.

* central finite differences of the forward `attend` (a plain softmax
  attention pinned elsewhere) against every gradient entry;
* torch autograd in float64 on the CPU, over a batch whose tokens share rows;
* invariants that hold at any size: the softmax gradient sums to zero over
  the keys (so the key gradients of one token sum to zero), the value
  gradients of one token sum to its upstream gradient, and one selected key
  passes no gradient to q or k;
* the log-sum-exp against scipy's.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O


def _rand(seed, n_sel=7, Hq=4, Hkv=2, D=8, mag=1.5):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(Hq, D)) * mag
    K = rng.normal(size=(n_sel, Hkv, D)) * mag
    V = rng.normal(size=(n_sel, Hkv, D))
    dO = rng.normal(size=(Hq, D))
    return q, K, V, dO


@pytest.mark.parametrize("seed,Hq,Hkv", [(0, 4, 2), (1, 4, 1), (2, 3, 3), (3, 8, 2)])
def test_backward_against_finite_differences(seed, Hq, Hkv):
    q, K, V, dO = _rand(seed, Hq=Hq, Hkv=Hkv)
    scale = 0.7
    dq, dK, dV = O.attend_backward(q, K, V, dO, Hkv, scale)

    def loss(q_, K_, V_):
        return float((O.attend(q_, K_, V_, Hkv, scale) * dO).sum())

    eps = 1e-6
    for name, X, G in (("q", q, dq), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        for ix in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[ix] += eps
            Xm[ix] -= eps
            args_p = {"q": q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            num[ix] = (loss(args_p["q"], args_p["K"], args_p["V"]) -
                       loss(args_m["q"], args_m["K"], args_m["V"])) / (2 * eps)
        assert np.abs(num - G).max() <= 1e-7 * max(1.0, np.abs(G).max()), name


def test_batch_backward_against_torch_autograd():
    rng = np.random.default_rng(5)
    T, n, Hq, Hkv, D = 40, 9, 4, 2, 16
    Q = rng.normal(size=(n, Hq, D))
    Kc = rng.normal(size=(T, Hkv, D))
    Vc = rng.normal(size=(T, Hkv, D))
    dO = rng.normal(size=(n, Hq, D))
    # overlapping selections, different lengths, one single-row selection
    rows = [np.sort(rng.choice(T, size=k, replace=False)) for k in (1, 5, 12, 40, 7, 7, 20, 3, 33)]
    scale = 1.0 / np.sqrt(D)
    dQ, dK, dV = O.sparse_attention_backward(Q, Kc, Vc, dO, rows, Hkv)

    tQ = torch.tensor(Q, requires_grad=True)
    tK = torch.tensor(Kc, requires_grad=True)
    tV = torch.tensor(Vc, requires_grad=True)
    total = torch.zeros((), dtype=torch.float64)
    for i, r in enumerate(rows):
        ri = torch.tensor(r)
        for h in range(Hq):
            g = h * Hkv // Hq
            k = tK[ri, g, :]
            v = tV[ri, g, :]
            w = torch.softmax((k @ tQ[i, h]) * scale, dim=0)
            total = total + ((w @ v) * torch.tensor(dO[i, h])).sum()
    total.backward()
    np.testing.assert_allclose(dQ, tQ.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tK.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tV.grad.numpy(), rtol=0, atol=1e-12)
    # rows nobody selected get zero
    unused = np.setdiff1d(np.arange(T), np.concatenate(rows))
    assert (dK[unused] == 0).all() and (dV[unused] == 0).all()


def test_backward_invariants():
    q, K, V, dO = _rand(9, n_sel=30, Hq=8, Hkv=2, D=16)
    dq, dK, dV = O.attend_backward(q, K, V, dO, 2)
    G = 4
    for g in range(2):
        # sum_j ds_j = 0 for every head  =>  the key gradients sum to zero
        assert np.abs(dK[:, g, :].sum(0)).max() <= 1e-12 * np.abs(dK).max() * 30
        # sum_j p_j = 1  =>  the value gradients sum to the heads' upstream gradients
        np.testing.assert_allclose(dV[:, g, :].sum(0), dO[g * G:(g + 1) * G].sum(0), atol=1e-12)
    # one key: p = 1, nothing flows to q or k; v gets the upstream gradient
    dq1, dK1, dV1 = O.attend_backward(q, K[:1], V[:1], dO, 2)
    assert np.abs(dq1).max() == 0 and np.abs(dK1).max() == 0
    np.testing.assert_allclose(dV1[0, 0], dO[:4].sum(0), atol=1e-14)
    # a duplicated row receives the gradient of both entries, which equals one entry of it
    # counted with doubled weight; the sum over the copies matches the merged row
    Kd = np.concatenate([K[:3], K[2:3]])
    Vd = np.concatenate([V[:3], V[2:3]])
    _, dKd, dVd = O.attend_backward(q, Kd, Vd, dO, 2)
    assert np.allclose(dKd[2], dKd[3]) and np.allclose(dVd[2], dVd[3])


def test_lse_against_scipy():
    q, K, V, dO = _rand(11, n_sel=25, Hq=6, Hkv=3, D=12, mag=3.0)
    out, lse = O.attend_lse(q, K, V, 3, 0.4)
    assert np.array_equal(out, O.attend(q, K, V, 3, 0.4))
    for h in range(6):
        g = h * 3 // 6
        assert abs(lse[h] - logsumexp(0.4 * (K[:, g, :] @ q[h]))) <= 1e-12
    _, lse1 = O.attend_lse(q, K[:1], V[:1], 3, 0.4)
    assert np.allclose(lse1, [0.4 * K[0, h * 3 // 6] @ q[h] for h in range(6)], atol=1e-14)


def test_stored_output_variant_equals_exact_when_given_the_exact_output():
    q, K, V, dO = _rand(13, n_sel=20, Hq=4, Hkv=2, D=16)
    o = O.attend(q, K, V, 2)
    a = O.attend_backward(q, K, V, dO, 2)
    b = O.attend_backward(q, K, V, dO, 2, o=o)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12 * max(1.0, np.abs(x).max())
    # a perturbed stored output moves dq and dK, never dV
    c = O.attend_backward(q, K, V, dO, 2, o=o + 1e-3)
    assert np.abs(c[0] - a[0]).max() > 1e-6 and np.abs(c[1] - a[1]).max() > 1e-6
    assert np.array_equal(c[2], a[2])


def test_round_bf16_against_torch_on_float32_values():
    rng = np.random.default_rng(17)
    x = (rng.normal(size=200000) * 10.0 ** rng.uniform(-20, 20, 200000)).astype(np.float32)
    x[:4] = [0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)]   # exact ties
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), want)
    assert O.round_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0            # tie to even
    assert O.round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
