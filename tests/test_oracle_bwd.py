"""Pins for the fp64 backward oracle (oracle.attention_backward), checked
against things other than its own formulas.

* finite differences: central differences of the forward oracle's loss
  sum(O * dO) with respect to every element of Q, K and V (tiny shapes, plain
  and causal) - the definition of the gradient, independent of the chain-rule
  algebra;
* library special case: torch autograd in float64 on the CPU through a plain
  torch expression of the definition (someone else's differentiation);
* closed forms: the keys' dK sum to zero (rows of dS sum to zero), the keys'
  dV sum to the queries' dO (rows of P sum to one), dO = 0 gives zero
  gradients, scale = 0 gives dQ = dK = 0 and dV_j = mean_i dO_i, N = 1 gives
  dQ = dK = 0 and dV = dO, causal row 0 gets dQ_0 = 0 (it sees one key);
* planted mistakes in the chain rule each fail at least one pin.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd_mod


def _rand(B, H, N, d, seed):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((B, H, N, d)) for _ in range(4))


def _bwd(q, k, v, do, scale, causal=False):
    return oracle.attention_backward(q, k, v, do, scale, causal=causal, workers=1)


def pin_finite_differences(bwd):
    for causal in (False, True):
        q, k, v, g = _rand(1, 2, 5, 3, 11 + causal)
        scale, h = 0.7, 1e-6
        dq, dk, dv = bwd(q, k, v, g, scale, causal)

        def loss(q_, k_, v_):
            o, _ = oracle.attention(q_, k_, v_, scale, causal=causal, workers=1)
            return float((o * g).sum())

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8,
                                       err_msg=f"d{name} causal={causal}")


def pin_torch_autograd(bwd):
    for causal in (False, True):
        q, k, v, g = _rand(2, 2, 9, 4, 21 + causal)
        scale = -0.4
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(9, 9, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(g))
        dq, dk, dv = bwd(q, k, v, g, scale, causal)
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def pin_closed_forms(bwd):
    q, k, v, g = _rand(2, 3, 17, 8, 31)
    dq, dk, dv = bwd(q, k, v, g, 0.35)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), g.sum(axis=2), rtol=1e-12, atol=1e-12)
    z = bwd(q, k, v, np.zeros_like(g), 0.35)
    for x in z:
        assert np.all(x == 0.0)
    dq0, dk0, dv0 = bwd(q, k, v, g, 0.0)
    assert np.all(dq0 == 0.0) and np.all(dk0 == 0.0)
    np.testing.assert_allclose(dv0, np.broadcast_to(g.mean(axis=2, keepdims=True), dv0.shape),
                               rtol=1e-12, atol=1e-12)
    q1, k1, v1, g1 = _rand(1, 2, 1, 8, 32)
    d1 = bwd(q1, k1, v1, g1, 0.9)
    np.testing.assert_allclose(d1[0], 0.0, atol=1e-13)
    np.testing.assert_allclose(d1[1], 0.0, atol=1e-13)
    np.testing.assert_allclose(d1[2], g1, rtol=1e-15)
    qc, kc, vc, gc = _rand(1, 2, 12, 8, 33)
    dqc, dkc, dvc = bwd(qc, kc, vc, gc, 0.5, True)
    np.testing.assert_allclose(dqc[:, :, 0], 0.0, atol=1e-13)      # row 0 sees one key
    np.testing.assert_allclose(dkc.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dvc.sum(axis=2), gc.sum(axis=2), rtol=1e-12, atol=1e-12)


PINS = [pin_finite_differences, pin_torch_autograd, pin_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pinned(pin):
    pin(_bwd)


def test_backward_row_chunking_changes_nothing():
    q, k, v, g = _rand(1, 2, 300, 16, 41)
    a = oracle.attention_backward(q, k, v, g, 0.2, workers=1, row_chunk=256)
    b = oracle.attention_backward(q, k, v, g, 0.2, workers=3, row_chunk=37)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def _planted(kind):
    """A copy of the per-head backward with one mistake."""
    def head(q, k, v, do, scale, causal, row_chunk):
        N = q.shape[0]
        s = scale * (q @ k.T)
        if causal:
            s[np.arange(N)[None, :] > np.arange(N)[:, None]] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v
        dv = (p @ do) if kind == "dv_no_transpose" else (p.T @ do)
        dp = do @ v.T
        dd = (do * o).sum(axis=1, keepdims=True)
        if kind == "no_D":
            ds = p * dp
        elif kind == "D_sign":
            ds = p * (dp + dd)
        else:
            ds = p * (dp - dd)
        dq = (ds @ k) * (1.0 if kind == "dq_no_scale" else scale)
        dk = scale * ((ds @ q) if kind == "dk_no_transpose" else (ds.T @ q))
        if kind == "dq_uses_v":
            dq = scale * (ds @ v)
        if kind == "causal_ignored_in_dv" and causal:
            pf = np.exp(scale * (q @ k.T))
            pf /= pf.sum(axis=1, keepdims=True)
            dv = pf.T @ do
        return dq, dk, dv
    return head


@pytest.mark.parametrize("kind", ["dv_no_transpose", "no_D", "D_sign", "dq_no_scale",
                                  "dk_no_transpose", "dq_uses_v", "causal_ignored_in_dv"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(bwd_mod, "_head_backward", _planted(kind))
    failed = 0
    for pin in PINS:
        try:
            pin(_bwd)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"planted mistake {kind} passed every pin"
