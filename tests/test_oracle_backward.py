"""Pins of the oracle's backward (gradients of sum(o * dO)): a hand-worked
example and central finite differences of the oracle forward on tiny inputs,
for every input, rate mode, momentum setting and both readout modes."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ttt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_backward_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_backward_T2.json")))
    sh = (1, 1, 2, 1)
    arr = lambda n: np.array(g[n], float).reshape(sh)
    eta = np.array(g["eta"], float).reshape(1, 1, 2)
    dq, dk, dv, de = oracle.backward(arr("q"), arr("k"), arr("v"), arr("dO"), eta_mode="per_token", eta=eta,
                                     beta=g["beta"])
    np.testing.assert_allclose(dq.ravel(), g["dq"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk.ravel(), g["dk"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.ravel(), g["dv"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(de.ravel(), g["deta"], rtol=0, atol=1e-12)


def _fd(f, x, h=1e-6):
    """Central finite differences of scalar f at every element of x."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy()
        xm = x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("eta_mode", ["scalar", "per_token", "softplus"])
@pytest.mark.parametrize("beta", [0.0, 0.7])
def test_backward_matches_finite_differences(causal, eta_mode, beta):
    rng = np.random.default_rng(21)
    B, H, T, dk_, dv_ = 1, 2, 4, 3, 2
    q = rng.standard_normal((B, H, T, dk_))
    k = rng.standard_normal((B, H, T, dk_))
    v = rng.standard_normal((B, H, T, dv_))
    dO = rng.standard_normal((B, H, T, dv_))
    a = rng.standard_normal((B, H, T))
    es = 0.8
    kw = dict(eta_mode=eta_mode, beta=beta, causal=causal)
    eta = None if eta_mode == "scalar" else a

    def L(q_=q, k_=k, v_=v, a_=eta, es_=es):
        return float((oracle.forward(q_, k_, v_, eta=a_, eta_scalar=es_, **kw) * dO).sum())

    dq, dk, dv, de = oracle.backward(q, k, v, dO, eta=eta, eta_scalar=es, **kw)
    np.testing.assert_allclose(dq, _fd(lambda x: L(q_=x), q), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dk, _fd(lambda x: L(k_=x), k), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dv, _fd(lambda x: L(v_=x), v), rtol=1e-6, atol=1e-7)
    if eta_mode == "scalar":
        fd = (L(es_=es + 1e-6) - L(es_=es - 1e-6)) / 2e-6
        assert abs(de - fd) <= 1e-6 * max(1.0, abs(fd))
    else:
        np.testing.assert_allclose(de, _fd(lambda x: L(a_=x), a), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("mistake", ["no_momentum_carry", "readout_grad_not_accumulated"])
def test_planted_backward_mistakes_fail_a_pin(monkeypatch, mistake):
    # a mistake planted in the adjoint recurrence fails the hand-worked pin
    test_backward_hand_example()
    orig = O.backward

    def bad(q, k, v, dO, **kw):
        if mistake == "no_momentum_carry":
            return orig(q, k, v, dO, **dict(kw, beta=0.0))
        # only each token's own readout feeds its state gradient
        T = np.shape(q)[2]
        outs = [orig(q[:, :, : t + 1], k[:, :, : t + 1], v[:, :, : t + 1],
                     np.concatenate([np.zeros_like(dO[:, :, :t]), dO[:, :, t:t + 1]], axis=2),
                     **dict(kw, eta=None if kw.get("eta") is None else kw["eta"][:, :, : t + 1]))
                for t in range(T)]
        return tuple(np.concatenate([o[i][:, :, -1:] for o in outs], axis=2) for i in range(3)) + (
            np.concatenate([o[3][:, :, -1:] for o in outs], axis=2),)

    monkeypatch.setattr(oracle, "backward", bad)
    with pytest.raises(AssertionError):
        test_backward_hand_example()


# ----------------------------------------------------------------------------
# SwiGLU feature map (Variant 2): gradients through phi and of W1, W3
# ----------------------------------------------------------------------------

def test_swiglu_backward_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_swiglu_backward_T1.json")))
    one = lambda x: np.full((1, 1, 1, 1), float(x))
    w = lambda x: np.full((1, 1, 1), float(x))
    o = oracle.forward(one(g["q"]), one(g["k"]), one(g["v"]), eta_mode="per_token", eta=np.full((1, 1, 1), g["eta"]),
                       phi="swiglu", w1=w(g["w1"]), w3=w(g["w3"]))
    assert abs(o.item() - g["o"]) <= 1e-12
    dq, dk, dv, de, dW1, dW3 = oracle.backward(one(g["q"]), one(g["k"]), one(g["v"]), one(g["dO"]),
                                               eta_mode="per_token", eta=np.full((1, 1, 1), g["eta"]),
                                               phi="swiglu", w1=w(g["w1"]), w3=w(g["w3"]))
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (de, "deta"), (dW1, "dW1"), (dW3, "dW3")):
        assert abs(np.asarray(got).item() - g[name]) <= 1e-12, name


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("eta_mode,beta", [("scalar", 0.0), ("softplus", 0.6), ("per_token", 0.6)])
def test_swiglu_backward_matches_finite_differences(causal, eta_mode, beta):
    rng = np.random.default_rng(22)
    B, H, T, d_in, d_phi, dv_ = 2, 2, 4, 3, 5, 2
    q = rng.standard_normal((B, H, T, d_in))
    k = rng.standard_normal((B, H, T, d_in))
    v = rng.standard_normal((B, H, T, dv_))
    dO = rng.standard_normal((B, H, T, dv_))
    a = rng.standard_normal((B, H, T))
    w1 = rng.standard_normal((H, d_phi, d_in)) * 0.7
    w3 = rng.standard_normal((H, d_phi, d_in)) * 0.7
    es = 0.8
    eta = None if eta_mode == "scalar" else a
    kw = dict(eta_mode=eta_mode, beta=beta, causal=causal, phi="swiglu")

    def L(q_=q, k_=k, v_=v, a_=eta, w1_=w1, w3_=w3):
        return float((oracle.forward(q_, k_, v_, eta=a_, eta_scalar=es, w1=w1_, w3=w3_, **kw) * dO).sum())

    dq, dk, dv, de, dW1, dW3 = oracle.backward(q, k, v, dO, eta=eta, eta_scalar=es, w1=w1, w3=w3, **kw)
    tol = dict(rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dq, _fd(lambda x: L(q_=x), q), **tol)
    np.testing.assert_allclose(dk, _fd(lambda x: L(k_=x), k), **tol)
    np.testing.assert_allclose(dv, _fd(lambda x: L(v_=x), v), **tol)
    np.testing.assert_allclose(dW1, _fd(lambda x: L(w1_=x), w1), **tol)
    np.testing.assert_allclose(dW3, _fd(lambda x: L(w3_=x), w3), **tol)
    if eta_mode != "scalar":
        np.testing.assert_allclose(de, _fd(lambda x: L(a_=x), a), **tol)


@pytest.mark.parametrize("mistake", ["silu_grad_as_sigmoid", "gate_grad_dropped"])
def test_planted_swiglu_backward_mistakes_fail_a_pin(monkeypatch, mistake):
    test_swiglu_backward_hand_example()
    if mistake == "silu_grad_as_sigmoid":
        monkeypatch.setattr(O, "silu_grad", lambda u: 1.0 / (1.0 + np.exp(-np.asarray(u, float))))
    else:
        orig = O.silu
        # the gate's own gradient dg = dphi * silu(u) lost: silu reads as zero where the
        # backward calls it

        def silu_only_in_forward(u):
            import inspect
            if inspect.stack()[1].function == "backward":
                return np.zeros_like(np.asarray(u, float))
            return orig(u)
        monkeypatch.setattr(O, "silu", silu_only_in_forward)
    with pytest.raises(AssertionError):
        test_swiglu_backward_hand_example()
